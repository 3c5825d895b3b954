"""The C-ABI library loads, exports every declared symbol, and its host-side
checks work without a GPU (no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from invariant_rmsnorm_backward_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return binding.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:rmsnorm|det_gemm|det_embedding)_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("rmsnorm_fwd", "rmsnorm_bwd_dx", "rmsnorm_dw_contrib", "rmsnorm_dw_finalize",
              "det_gemm_bwd_dx", "det_gemm_dw_contrib", "det_gemm_dw_finalize"):
        assert n in names
    assert sorted(binding.EXPORTED) == names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_backend_info_names_the_order(lib):
    info = binding.rmsnorm_backend_info()
    assert "gfx950" in info and "cdo=v2" in info and "no atomics" in info
    assert binding.rmsnorm_max_hidden() >= 8192


def test_layout_check_stats_and_errors(lib):
    # hidden-independent plan: 59 rows padded to 80, permuted samples
    rl = np.full(80, -1, dtype=np.int32)
    rl[10:69] = np.random.default_rng(0).permutation(59)
    st = binding.rmsnorm_layout_check(rl, 59)
    assert st == {"blocks": 1, "complete_blocks": 1, "partial_blocks": 0, "pad_rows": 21,
                  "real_rows": 59}
    # a chunk holding rows 60..129 of 200: blocks 0 and 2 in part, block 1 whole
    st = binding.rmsnorm_layout_check(np.arange(60, 130, dtype=np.int32), 200)
    assert st["blocks"] == 3 and st["partial_blocks"] == 2 and st["complete_blocks"] == 1
    st = binding.rmsnorm_layout_check(np.arange(64, 128, dtype=np.int32), 200)
    assert st["complete_blocks"] == 1 and st["partial_blocks"] == 0
    # the last block is complete when it holds every present row (T = 70)
    st = binding.rmsnorm_layout_check(np.arange(64, 70, dtype=np.int32), 70)
    assert st["complete_blocks"] == 1
    for bad, code in (([0, 0], binding.ELAYOUT), ([0, 5], binding.ELAYOUT),
                      ([-2, 1], binding.ELAYOUT)):
        with pytest.raises(binding.RmsNormError) as ei:
            binding.rmsnorm_layout_check(np.array(bad, dtype=np.int32), 5)
        assert ei.value.code == code
        assert "logical" in ei.value.message or "outside" in ei.value.message


def test_argument_errors_are_refused_before_any_launch(lib):
    A = 1 << 20  # a fake, aligned address: never dereferenced because checks fail first
    cases = [
        (dict(hidden=12), binding.EUNSUPPORTED),
        (dict(hidden=0), binding.EINVAL),
        (dict(hidden=binding.rmsnorm_max_hidden() + 8), binding.EUNSUPPORTED),
        (dict(rows=-1), binding.EINVAL),
        (dict(eps=-1.0), binding.EINVAL),
        (dict(eps=float("nan")), binding.EINVAL),
        (dict(x=0), binding.EINVAL),
        (dict(x=A + 2), binding.EUNSUPPORTED),
        (dict(y=A), binding.EINVAL),                   # y aliases x
    ]
    for over, code in cases:
        args = dict(x=A, w=A + 4096 * 1024, y=A + 8192 * 1024, rstd=A + 12288 * 1024, rows=4,
                    hidden=4096, eps=1e-6)
        args.update(over)
        with pytest.raises(binding.RmsNormError) as ei:
            binding.rmsnorm_fwd(args["x"], args["w"], args["y"], args["rstd"], args["rows"],
                                args["hidden"], args["eps"], None, None)
        assert ei.value.code == code, (over, ei.value)
    with pytest.raises(binding.RmsNormError) as ei:
        binding.rmsnorm_dw_contrib(A, A, A, 4, 4096, None, None, None)
    assert ei.value.code == binding.EINVAL
    with pytest.raises(binding.RmsNormError) as ei:
        binding.rmsnorm_dw_finalize(None, A, None)
    assert ei.value.code == binding.EINVAL


def test_no_atomics_and_no_fallbacks_in_the_library_sources():
    csrc = os.path.join(ROOT, "invariant_rmsnorm_backward_amd", "csrc")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name)).read()
        code = re.sub(r"//.*", "", re.sub(r"/\*.*?\*/", "", text, flags=re.S))
        assert not re.search(r"\batomic\w*\s*\(|__atomic|std::atomic|__hip_atomic", code), name
        assert "__CUDA" not in code and "cuda_runtime" not in code, name
        assert "__HIP_PLATFORM" not in code, name
    # the kernel shapes (lane groups, wavefronts per row, chunks per lane,
    # rows in flight) key on the hidden size only
    k = open(os.path.join(csrc, "kernels.hip")).read()
    for ret, fn in (("int", "small_lanes"), ("int", "fwd_tw"), ("int", "fwd_v"),
                    ("BwdShape", "fused_shape"), ("BwdShape", "split_shape"),
                    ("BwdShape", "stream_shape")):
        sig = re.search(rf"static {ret} {fn}\(([^)]*)\)", k).group(1)
        assert sig.strip() == "int hidden", fn


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "invariant_rmsnorm_backward_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "liboracle" not in text, f


def test_split_threshold_knob():
    """The backward's work-distribution threshold: set, read back, restore."""
    prev = binding.rmsnorm_set_split_threshold(5)
    try:
        assert binding.rmsnorm_set_split_threshold(0) == 5
        assert binding.rmsnorm_set_split_threshold(-1) == 0      # negative: back to the default
        assert binding.rmsnorm_set_split_threshold(prev) > 0
    finally:
        binding.rmsnorm_set_split_threshold(prev)


def test_stream_threshold_knob():
    """The stream-owner backward's lower bound: set, read back, restore."""
    prev = binding.rmsnorm_set_stream_threshold(7)
    try:
        assert binding.rmsnorm_set_stream_threshold(0) == 7
        assert binding.rmsnorm_set_stream_threshold(-1) == 0     # negative: back to the default
        assert binding.rmsnorm_set_stream_threshold(prev) == 32
    finally:
        binding.rmsnorm_set_stream_threshold(prev)


def test_stream_copy_checks_its_arguments(lib):
    """The bandwidth-probe copy refuses bad arguments before touching the GPU."""
    A = 1 << 12
    cases = [((A, A + 4096, -16), binding.EINVAL),           # negative size
             ((0, A, 64), binding.EINVAL),                   # NULL source
             ((A, A + 4096, 40), binding.EUNSUPPORTED),      # not a multiple of 16
             ((A + 8, A + 8192, 64), binding.EUNSUPPORTED),  # misaligned
             ((A, A + 32, 64), binding.EINVAL)]              # overlapping ranges
    for (src, dst, n), code in cases:
        with pytest.raises(binding.RmsNormError) as ei:
            binding.rmsnorm_stream_copy(src, dst, n, None)
        assert ei.value.code == code, (src, dst, n)
    binding.rmsnorm_stream_copy(A, A + 4096, 0, None)       # zero bytes: a no-op


def test_stream_2r1w_checks_its_arguments(lib):
    """The two-read probe refuses bad arguments before touching the GPU."""
    A = 1 << 12
    cases = [((A, A + 4096, A + 8192, -16), binding.EINVAL),           # negative size
             ((A, 0, A + 8192, 64), binding.EINVAL),                   # NULL input
             ((A, A + 4096, A + 8192, 40), binding.EUNSUPPORTED),      # not a multiple of 16
             ((A, A + 4096, A + 8200, 64), binding.EUNSUPPORTED),      # misaligned output
             ((A, A + 4096, A + 4096 + 32, 64), binding.EINVAL)]       # output overlaps b
    for (a, b, c, n), code in cases:
        with pytest.raises(binding.RmsNormError) as ei:
            binding.rmsnorm_stream_2r1w(a, b, c, n, None)
        assert ei.value.code == code, (a, b, c, n)
    binding.rmsnorm_stream_2r1w(A, A, A + 4096, 0, None)      # zero bytes: a no-op


def test_workgroup_cap_knob():
    """The fused backward's workgroup cap: set, read back, restore."""
    prev = binding.rmsnorm_set_workgroup_cap(3)
    try:
        assert binding.rmsnorm_set_workgroup_cap(1) == 3
        assert binding.rmsnorm_set_workgroup_cap(-5) == 1       # negative: back to the default
        assert binding.rmsnorm_set_workgroup_cap(prev) == 0
    finally:
        binding.rmsnorm_set_workgroup_cap(prev)


def test_packed_entry_points_check_their_arguments(lib):
    A = 1 << 12
    cases = [
        (dict(head_dim=96), binding.EUNSUPPORTED),        # no packed kernel for 96
        (dict(token_stride=100), binding.EINVAL),         # not a multiple of 8
        (dict(token_stride=8), binding.EINVAL),           # shorter than heads * head_dim
        (dict(heads=0), binding.EINVAL),
        (dict(tokens=-1), binding.EINVAL),
    ]
    for over, code in cases:
        a = dict(tokens=4, heads=2, head_dim=128, token_stride=512)
        a.update(over)
        with pytest.raises(binding.RmsNormError) as ei:
            binding.rmsnorm_fwd_packed(A, A, A, A, a["tokens"], a["heads"], a["head_dim"],
                                       a["token_stride"], 1e-6, None, None)
        assert ei.value.code == code, over
    # zero tokens is a successful no-op
    binding.rmsnorm_fwd_packed(A, A, A, A, 0, 2, 128, 512, 1e-6, None, None)


def test_noalloc_refusals_before_any_launch(lib):
    """The allocation-free backward checks its sizes and pointers on the host:
    more block partials than its scratch holds, a NULL dweight, aliasing and a
    bad width are refused before anything is enqueued."""
    A = 1 << 20
    limit = binding.rmsnorm_bwd_noalloc_max_scratch()
    assert limit == 16 << 20
    # 16M floats hold 262,143 rows at hidden 4096 (plus the tree levels); refuse beyond
    too_many = (limit // 4096) * 64 + 64
    for args, code in (((A, A, A, A, A, A, too_many, 4096), binding.EUNSUPPORTED),
                       ((A, A, A, A, A, 0, 10, 4096), binding.EINVAL),
                       ((A, A, A, A, A, A, 10, 12), binding.EUNSUPPORTED),
                       ((A, A + (1 << 24), A + (2 << 24), A + (3 << 24), A, A + (4 << 24), 10, 4096),
                        binding.EINVAL),   # dx aliases x
                       ((A, A + (1 << 24), A + (2 << 24), A + (3 << 24), A + (4 << 24), A, 10, 4096),
                        binding.EINVAL)):  # dweight aliases x
        with pytest.raises(binding.RmsNormError) as ei:
            binding.rmsnorm_bwd_noalloc(*args, None)
        assert ei.value.code == code, (args, ei.value)


def test_packed_pair_checks_its_arguments(lib):
    """The one-launch Q/K pair refuses, before any launch, what either single
    call would refuse, outputs that share elements, and one accumulator for
    both norms; zero tokens is a no-op."""
    A = 1 << 24
    hd, hq, hk = 128, 4, 2
    ts = (hq + 2 * hk) * hd                      # elements per token
    tok = 4
    ext = ((tok - 1) * ts + hq * hd) * 2         # bytes a norm's rows span
    X, Y, DY, DX, W, R = A, A + (1 << 22), A + (2 << 22), A + (3 << 22), A + (4 << 22), A + (5 << 22)
    kcol = hq * hd * 2                           # byte offset of the K heads in a token

    def fwd(yk=Y + kcol, head_dim=hd, tokens=tok, stride_k=ts):
        a = (X, W, Y, R, hq, ts, None)
        b = (X + kcol, W + 4096, yk, R + 65536, hk, stride_k, None)
        binding.rmsnorm_fwd_packed_pair(a, b, tokens, head_dim, 1e-6, None)

    for kw, code in ((dict(head_dim=96), binding.EUNSUPPORTED),
                     (dict(yk=Y + 128), binding.EINVAL),          # K outputs inside the Q windows
                     (dict(yk=X + kcol), binding.EINVAL),         # K output on the pair's input
                     (dict(stride_k=100), binding.EINVAL)):       # not a multiple of 8
        with pytest.raises(binding.RmsNormError) as ei:
            fwd(**kw)
        assert ei.value.code == code, (kw, ei.value)
    fwd(tokens=0)                                # nothing to do
    ACC = 1 << 30                                # never dereferenced: refused first
    a = (X, W, DY, R, DX, hq, ts, None, ACC)
    b = (X + kcol, W + 4096, DY + kcol, R + 65536, DX + kcol, hk, ts, None, ACC)
    with pytest.raises(binding.RmsNormError) as ei:
        binding.rmsnorm_bwd_dx_packed_pair(a, b, tok, hd, None)
    assert ei.value.code == binding.EINVAL and "accumulators" in ei.value.message
    assert ext > 0
