"""C ABI on the CPU: the library loads, exports every function include/moe.h
declares, and its host-only calls (sizes, validation) behave -- no kernel is
launched here (every error below is caught before any HIP call)."""
import ctypes
import os
import re

import pytest

from bit_moe_expert_03_amd import binding as B
from bit_moe_expert_03_amd import workload as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)


def test_header_lists_the_binding_exports():
    assert sorted(header_functions()) == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    assert B.moe_abi_version() == 5


def test_status_strings():
    L = B.lib()
    for st in range(5):
        assert L.moe_status_string(st)


@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_sizes_of_the_workloads(name):
    dm = B.make_dims(wl.CONFIGS[name])
    tm = B.moe_tile_m(dm)
    assert tm in (32, 64, 128)
    A = dm.T * dm.k
    assert B.moe_max_tiles(dm) == -(-A // tm) + min(dm.E, A)
    ws = B.moe_workspace_bytes(dm)
    # the workspace holds at least h (routed + shared) and the routed outputs
    assert ws >= A * dm.F * 2 + dm.T * dm.Fs * 2 + A * dm.d * 2


def test_valid_down_nc_is_accepted():
    """Every chain length that divides d/256 on a chainable shape is a valid
    schedule field; 0 and 1 are valid on every shape."""
    chain = wl.Dims(T=16, d=1024, E=16, k=2, F=128, Fs=128, G=32)
    for nc in (0, 1, 2, 4):
        assert B.moe_workspace_bytes(B.make_dims(chain, down_nc=nc)) > 0
    for nc in (0, 1):
        assert B.moe_workspace_bytes(B.make_dims(wl.CONFIGS["c0_tiny"], down_nc=nc)) > 0


def test_explicit_tile_m_is_kept():
    for tm in (32, 64, 128):
        dm = B.make_dims(wl.CONFIGS["c2_prefill512"], tile_m=tm)
        assert B.moe_tile_m(dm) == tm


BAD = [
    dict(E=0), dict(E=257), dict(k=0), dict(k=17), dict(G=16), dict(d=96), dict(F=100),
    dict(Fs=0), dict(T=-1), dict(tile_m=48), dict(d=64 * 300),
    # down-GEMM chain lengths that do not fit the shape (d = 256: one column block)
    dict(down_nc=-1), dict(down_nc=65), dict(down_nc=2), dict(d=512, down_nc=4),
    dict(d=512, F=192, Fs=192, G=64, down_nc=2), dict(d=512, Fs=256, down_nc=2),
    # activation matrices of 2^31 elements or more (32-bit byte offsets)
    dict(T=1 << 20, d=2048), dict(T=1 << 20, k=8, F=256), dict(T=1 << 20, Fs=2048),
]


@pytest.mark.parametrize("bad", BAD, ids=[str(b) for b in BAD])
def test_invalid_dims_are_rejected_without_launch(bad):
    base = dict(T=16, d=256, E=16, k=2, F=128, Fs=128, G=32, tile_m=0, down_nc=0)
    base.update(bad)
    dm = B.moe_dims(**base)
    assert B.moe_tile_m(dm) == 0 and B.moe_max_tiles(dm) == 0 and B.moe_workspace_bytes(dm) == 0
    r = B.moe_routing()
    st = B.lib().moe_route(ctypes.byref(dm), None, ctypes.byref(r), None, 0, None)
    assert st == B.MOE_ERR_SHAPE
    assert B.lib().moe_last_error()


def _fake_ptr(i):
    # distinct aligned non-null host addresses: never dereferenced, since every
    # call below fails validation before anything is launched
    return 0x10000000 + 0x100000 * i


def test_null_pointers_and_small_workspace_are_rejected():
    L = B.lib()
    dm = B.make_dims(wl.CONFIGS["c0_tiny"])
    need = B.moe_workspace_bytes(dm)
    r = B.moe_routing(*[_fake_ptr(i) for i in range(10)])
    # workspace too small
    st = L.moe_route(ctypes.byref(dm), _fake_ptr(20), ctypes.byref(r), _fake_ptr(21), need - 1, None)
    assert st == B.MOE_ERR_WORKSPACE
    # null logits
    st = L.moe_route(ctypes.byref(dm), None, ctypes.byref(r), _fake_ptr(21), need, None)
    assert st == B.MOE_ERR_ARG
    # misaligned routing pointer
    r2 = B.moe_routing(*[_fake_ptr(i) for i in range(10)])
    r2.perm = _fake_ptr(4) + 4
    st = L.moe_route(ctypes.byref(dm), _fake_ptr(20), ctypes.byref(r2), _fake_ptr(21), need, None)
    assert st == B.MOE_ERR_ARG
    # ffn: null weight pointer, x/y overlap
    w = B.moe_weights(*[B.moe_qmat(_fake_ptr(30 + 3 * i), _fake_ptr(31 + 3 * i), _fake_ptr(32 + 3 * i))
                        for i in range(6)])
    w.down.q = None
    st = L.moe_ffn(ctypes.byref(dm), _fake_ptr(50), ctypes.byref(w), ctypes.byref(r), _fake_ptr(51),
                   _fake_ptr(21), need, None)
    assert st == B.MOE_ERR_ARG and b"down" in L.moe_last_error()
    w.down.q = _fake_ptr(36)
    st = L.moe_ffn(ctypes.byref(dm), _fake_ptr(50), ctypes.byref(w), ctypes.byref(r), _fake_ptr(50) + 256,
                   _fake_ptr(21), need, None)
    assert st == B.MOE_ERR_ARG and b"overlap" in L.moe_last_error()
    # dequant: bad G, bad cols
    q = B.moe_qmat(_fake_ptr(60), _fake_ptr(61), _fake_ptr(62))
    assert L.moe_dequant(ctypes.byref(q), 4, 64, 48, _fake_ptr(63), None) == B.MOE_ERR_SHAPE
    assert L.moe_dequant(ctypes.byref(q), 4, 48, 32, _fake_ptr(63), None) == B.MOE_ERR_SHAPE


def test_kernel_counts_of_each_path():
    """1 <= T <= 32 with T*k <= 512: two kernels (decode gate/up with routing,
    decode down); larger batches: three routing kernels and three GEMM-path
    kernels; T = 0: one."""
    base = dict(d=256, E=128, F=128, Fs=128, G=64)
    for T, k, n in [(1, 8, 2), (1, 17, 2), (2, 8, 2), (8, 8, 2), (8, 64, 2), (9, 8, 2), (8, 65, 6),
                    (16, 8, 2), (32, 16, 2), (32, 17, 6), (33, 8, 6), (4096, 8, 6), (0, 8, 1)]:
        dm = B.make_dims(wl.Dims(T=T, k=k, **base))
        assert B.moe_layer_kernels(dm) == n, (T, k)


def test_router_packed_bytes_and_argument_checks():
    """Packed router size: two bf16 matrices of roundup(E, 64) rows x d; the
    router entry points reject null pointers before launching anything."""
    dm = B.make_dims(wl.CONFIGS["c1_decode"])
    assert B.moe_router_packed_bytes(dm) == 2 * 256 * 2048 * 2
    dm16 = B.make_dims(wl.CONFIGS["c0_tiny"])
    assert B.moe_router_packed_bytes(dm16) == 2 * 64 * 256 * 2
    L = B.lib()
    assert L.moe_router_pack(ctypes.byref(dm), None, None, None) == B.MOE_ERR_ARG
    r = B.moe_routing()
    assert L.moe_route_x(ctypes.byref(dm), None, None, None, None, ctypes.byref(r), None,
                         B.moe_workspace_bytes(dm), None) == B.MOE_ERR_ARG
    bad = B.make_dims(wl.CONFIGS["c1_decode"].replace(E=0))
    assert B.moe_router_packed_bytes(bad) == 0


def test_noalloc_entry_point_rejects_before_any_device_call():
    """moe_layer_noalloc: dims whose workspace exceeds its scratch array
    (T = 4096: about 213 MiB against 32 MiB) and null pointers are refused on
    the host, before the scratch address is looked up or anything launched."""
    L = B.lib()
    big = B.make_dims(wl.CONFIGS["c3_prefill4096_zipf"])
    assert B.moe_workspace_bytes(big) > B.NOALLOC_SCRATCH_BYTES
    r = B.moe_routing(*[_fake_ptr(i) for i in range(10)])
    w = B.moe_weights(*[B.moe_qmat(_fake_ptr(30 + 3 * i), _fake_ptr(31 + 3 * i), _fake_ptr(32 + 3 * i))
                        for i in range(6)])
    st = L.moe_layer_noalloc(ctypes.byref(big), _fake_ptr(20), _fake_ptr(50), ctypes.byref(w), ctypes.byref(r),
                             _fake_ptr(51), None)
    assert st == B.MOE_ERR_WORKSPACE and L.moe_last_error()
    small = B.make_dims(wl.CONFIGS["c0_tiny"])
    assert B.moe_workspace_bytes(small) <= B.NOALLOC_SCRATCH_BYTES
    st = L.moe_layer_noalloc(ctypes.byref(small), None, _fake_ptr(50), ctypes.byref(w), ctypes.byref(r),
                             _fake_ptr(51), None)
    assert st == B.MOE_ERR_ARG


def test_noalloc_limit_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES


def test_gqa_workspace_and_argument_checks():
    """Decode attention: workspace holds fp32 (o, max, sum) per split and
    query head; unsupported dims give 0 bytes and MOE_ERR_SHAPE, null,
    misaligned or overlapping pointers and a small workspace are refused
    before anything is launched."""
    L = B.lib()
    a = B.make_attn_dims(wl.ATTN_CONFIGS["attn_L32768"])
    need = B.moe_gqa_workspace_bytes(a)
    # bound over every device: min(1024, ceil(L / 64)) splits of (o, max, sum) per query head
    assert need == 512 * 32 * (128 + 2) * 4
    assert B.moe_gqa_workspace_bytes(B.moe_attn_dims(32, 4, 128, 1)) == 1 * 32 * 130 * 4
    for bad in [(33, 4, 128, 64), (32, 4, 96, 64), (32, 4, 128, 0), (0, 0, 128, 64), (8 * 129, 129, 64, 8),
                (32, 4, 128, (1 << 24) + 1)]:
        d = B.moe_attn_dims(*bad)
        assert B.moe_gqa_workspace_bytes(d) == 0, bad
        st = L.moe_gqa_decode(ctypes.byref(d), _fake_ptr(1), _fake_ptr(2), _fake_ptr(3), _fake_ptr(4),
                              _fake_ptr(5), 1 << 30, None)
        assert st == B.MOE_ERR_SHAPE, bad
    assert L.moe_gqa_decode(None, None, None, None, None, None, 0, None) == B.MOE_ERR_ARG
    args = [_fake_ptr(i) for i in range(1, 6)]
    for i in range(5):
        for broken in (None, args[i] + 4):
            t = list(args)
            t[i] = broken
            assert L.moe_gqa_decode(ctypes.byref(a), *t, need, None) == B.MOE_ERR_ARG, (i, broken)
    assert L.moe_gqa_decode(ctypes.byref(a), *args, need - 1, None) == B.MOE_ERR_WORKSPACE
    # o inside k
    kv = 4 * 32768 * 128 * 2
    t = list(args)
    t[3] = args[1] + kv - 256
    assert L.moe_gqa_decode(ctypes.byref(a), *t, need, None) == B.MOE_ERR_ARG
    assert b"overlap" in L.moe_last_error()
    ev = (ctypes.c_void_p * 3)()
    assert L.moe_gqa_decode_timed(ctypes.byref(a), *args, need, None, ev, 3) == B.MOE_ERR_ARG


def test_fewrow_parity_cases_have_fewrow_experts():
    """The GPU parity cases named fewrow_* route many experts to one or two
    rows and some to three or more."""
    import oracle
    import test_gpu_parity as P
    for name, (dims, zipf) in P.SMALL.items():
        if not name.startswith("fewrow_"):
            continue
        c = wl.make_case(dims, seed=100 + list(P.SMALL).index(name), zipf=zipf, weights=False)
        counts = oracle.route(c["logits"], dims.k, 32)["counts"]
        assert ((counts >= 1) & (counts <= 2)).sum() >= 10, name
        assert (counts >= 3).sum() >= 1, name
