"""C ABI checks that need no GPU: the library loads, exports every function
include/tq_decode.h declares, and rejects bad arguments on the host before
touching the device.  Every call made here fails validation, so no kernel is
ever enqueued."""

import ctypes
import os
import re

import pytest

import paged_gqa_decode_amd as tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq_decode.h")
PROBE_HEADER = os.path.join(ROOT, "include", "tq_probe.h")


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(tq4?_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return tq.load_library()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(tq.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_probe_library_exports_its_header():
    from paged_gqa_decode_amd import probe

    names = header_functions(PROBE_HEADER)
    assert set(names) == set(probe.EXPORTED_SYMBOLS), names
    plib = probe.load_library()
    for n in names:
        assert hasattr(plib, n), f"{n} not exported"
    # argument errors are reported without touching the device
    assert plib.tq_probe_read(0, 16, 0x10000, 1, None) != 0
    assert plib.tq_probe_copy(0x10000, 0x10000, 17, 1, None) != 0
    assert plib.tq_probe_pattern4(0, 0x10000, 4096, 256, 1, 1, 0x10000, None) != 0
    assert plib.tq_probe_pattern4(0x10000, 0x10000, 4095, 256, 1, 1, 0x10000, None) != 0


def test_every_header_is_covered():
    hdrs = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert hdrs == ["tq_decode.h", "tq_probe.h"], hdrs


def test_abi_version_and_status_strings(lib):
    assert tq.abi_version() == 2
    for st in range(9):
        assert tq.status_str(st) != "unknown status"
    assert tq.status_str(99) == "unknown status"
    assert tq.last_hip_error() == 0


def test_partials_bytes(lib):
    # rows = S*Hkv*P*QG; out fp32 128 per row, two fp32 arrays, each rounded to 256 B
    rows = 128 * 8 * 32 * 8
    assert tq.partials_bytes(128, 8, 32, 8) == rows * 512 + 2 * rows * 4
    assert tq.partials_bytes(1, 1, 1, 6) == 3072 + 2 * 256
    assert tq.partials_bytes(1, 1, 1, 7) == 0
    assert tq.partials_bytes(0, 1, 1, 8) == 0


# Fake, aligned, non-null addresses: only ever passed to calls that must fail validation.
A = 0x10000


def call_decode(lib, *, ptrs=None, QG=8, BS=16, G=1, Hkv=2, scale=0.088, S=2, NB=8, MB=4, P=1,
                maxlen=64, head_dim=128, part=None, layout=0):
    ptrs = ptrs or [A] * 6
    ps = tq.PartialsStruct(*(part or (A, A, A)))
    ext = tq.Extent(S, NB, MB, P, maxlen, head_dim, layout)
    return lib.tq_decode(*ptrs, ctypes.byref(ps), Hkv, QG, BS, G, scale, ctypes.byref(ext), None)


@pytest.mark.parametrize("kw,status", [
    (dict(ptrs=[0, A, A, A, A, A]), tq.TQ_ERR_NULL),
    (dict(ptrs=[A, A, A, A, A, 0]), tq.TQ_ERR_NULL),
    (dict(part=(A, 0, A)), tq.TQ_ERR_NULL),
    (dict(QG=7), tq.TQ_ERR_UNSUPPORTED),
    (dict(QG=4), tq.TQ_ERR_UNSUPPORTED),
    (dict(BS=8), tq.TQ_ERR_UNSUPPORTED),
    (dict(BS=64), tq.TQ_ERR_UNSUPPORTED),
    (dict(head_dim=64), tq.TQ_ERR_UNSUPPORTED),
    (dict(layout=2), tq.TQ_ERR_UNSUPPORTED),
    (dict(layout=-1), tq.TQ_ERR_UNSUPPORTED),
    (dict(S=0), tq.TQ_ERR_SHAPE),
    (dict(Hkv=0), tq.TQ_ERR_SHAPE),
    (dict(NB=0), tq.TQ_ERR_SHAPE),
    (dict(MB=0), tq.TQ_ERR_SHAPE),
    (dict(P=0), tq.TQ_ERR_SHAPE),
    (dict(G=0), tq.TQ_ERR_SHAPE),
    (dict(S=1 << 20, Hkv=1 << 8, P=1 << 8), tq.TQ_ERR_SHAPE),
    (dict(maxlen=-1), tq.TQ_ERR_COVERAGE),
    (dict(maxlen=257, P=1, MB=64), tq.TQ_ERR_COVERAGE),      # > P*256*G
    (dict(maxlen=65, P=1, MB=4), tq.TQ_ERR_COVERAGE),        # > max_blocks_per_seq*BS
    (dict(scale=0.0), tq.TQ_ERR_SCALE),
    (dict(scale=-1.0), tq.TQ_ERR_SCALE),
    (dict(scale=float("nan")), tq.TQ_ERR_SCALE),
    (dict(scale=float("inf")), tq.TQ_ERR_SCALE),
    (dict(ptrs=[A + 2, A, A, A, A, A]), tq.TQ_ERR_MISALIGNED),
    (dict(ptrs=[A, A + 8, A, A, A, A]), tq.TQ_ERR_MISALIGNED),
    (dict(ptrs=[A, A, A, A + 4, A, A]), tq.TQ_ERR_MISALIGNED),
    (dict(ptrs=[A, A, A, A, A + 2, A]), tq.TQ_ERR_MISALIGNED),
    (dict(part=(A + 4, A, A)), tq.TQ_ERR_MISALIGNED),
])
def test_decode_rejects(lib, kw, status):
    assert call_decode(lib, **kw) == status


def test_coverage_boundary_from_the_page_sizing_example(lib):
    """32 partitions x 5 tile groups x 256 tokens = 40960 tokens at block size 32."""
    import json
    fig = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))["sizing_example"]
    P, G, BS, covered = fig["num_partitions"], fig["tile_groups_per_partition"], fig["kv_block_size"], \
        fig["covered_tokens"]
    assert P * G * tq.TOKENS_PER_TILE_GROUP == covered
    # one token past the coverage is rejected; (at the coverage the call would launch, so
    # it is exercised only by the GPU tests)
    assert call_decode(lib, P=P, G=G, BS=BS, MB=covered // BS + 8, maxlen=covered + 1) == \
        tq.TQ_ERR_COVERAGE
    assert call_decode(lib, P=P, G=G, BS=BS, MB=covered // BS, maxlen=covered, scale=0.0) == \
        tq.TQ_ERR_SCALE  # coverage passes; the scale check then fails before any launch


def call_fused(lib, *, ptrs=None, out=A, QG=8, BS=16, G=1, Hkv=2, scale=0.088, S=2, NB=8, MB=4,
               P=1, maxlen=64, head_dim=128, ws=None, ws_bytes=0):
    ptrs = ptrs or [A] * 6
    ext = tq.Extent(S, NB, MB, P, maxlen, head_dim)
    return lib.tq_decode_fused(*ptrs, out, Hkv, QG, BS, G, scale, ctypes.byref(ext), ws, ws_bytes,
                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=0), tq.TQ_ERR_NULL),
    (dict(ptrs=[A, A, 0, A, A, A]), tq.TQ_ERR_NULL),
    (dict(QG=12), tq.TQ_ERR_UNSUPPORTED),
    (dict(BS=48), tq.TQ_ERR_UNSUPPORTED),
    (dict(P=0), tq.TQ_ERR_SHAPE),
    (dict(maxlen=300, P=1, MB=64), tq.TQ_ERR_COVERAGE),
    (dict(scale=float("nan")), tq.TQ_ERR_SCALE),
    (dict(out=A + 8), tq.TQ_ERR_MISALIGNED),
    (dict(ptrs=[A, A, A, A, A, A + 1]), tq.TQ_ERR_MISALIGNED),
    (dict(ws=A + 8, ws_bytes=1 << 20), tq.TQ_ERR_MISALIGNED),
])
def test_fused_rejects(lib, kw, status):
    assert call_fused(lib, **kw) == status


def _r256(x):
    return (x + 255) // 256 * 256


def _flat_bytes(seq_heads, groups, QG):
    rows = 2 * groups * QG  # two partial slots per workgroup
    return _r256(seq_heads * 4) + _r256(rows * 512) + 2 * _r256(rows * 4)


def test_fused_workspace_bytes():
    # the flat work list of 32-token entries: 256 workgroups of 8 waves once it has 2048
    assert tq.fused_workspace_bytes(128, 8, 8, 8192) == _flat_bytes(1024, 256, 8)
    assert tq.fused_workspace_bytes(16, 4, 16, 40960) == _flat_bytes(64, 256, 16)
    assert tq.fused_workspace_bytes(256, 1, 6, 256) == _flat_bytes(256, 256, 6)
    # a shorter list: at most one wave per entry (4 x 7 entries: four workgroups)
    assert tq.fused_workspace_bytes(4, 1, 16, 200) == _flat_bytes(4, 4, 16)
    assert tq.fused_workspace_bytes(1, 1, 8, 32) == _flat_bytes(1, 1, 8)
    assert tq.fused_workspace_bytes(16, 4, 7, 40960) == 0  # unsupported QG
    assert tq.fused_workspace_bytes(1024, 8, 8, 2048) == _flat_bytes(8192, 256, 8)
    # more than 1024 sequences: workgroups per (s, h) instead, split by the per-(s, h) plan
    assert tq.fused_workspace_bytes(1025, 8, 8, 8192) == 0   # 8200 (s, h): one workgroup each
    assert tq.fused_workspace_bytes(1025, 1, 8, 40960) == 0  # 1025 (s, h): one workgroup each


def call_tq4(lib, *, fused=False, q=A, cache=A, cent=A, bt=A, sl=A, out=A, QG=8, BS=16, G=1, Hkv=2,
             scale=0.088, S=2, NB=8, MB=4, P=1, maxlen=64, head_dim=128):
    ext = tq.Extent(S, NB, MB, P, maxlen, head_dim)
    if fused:
        return lib.tq4_decode_fused(q, cache, cent, bt, sl, out, Hkv, QG, BS, G, scale,
                                    ctypes.byref(ext), None, 0, None)
    ps = tq.PartialsStruct(out, A, A) if out else tq.PartialsStruct(0, A, A)
    return lib.tq4_decode(q, cache, cent, bt, sl, ctypes.byref(ps), Hkv, QG, BS, G, scale,
                          ctypes.byref(ext), None)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(cache=0), tq.TQ_ERR_NULL),
    (dict(cent=0), tq.TQ_ERR_NULL),
    (dict(q=0), tq.TQ_ERR_NULL),
    (dict(out=0), tq.TQ_ERR_NULL),
    (dict(QG=7), tq.TQ_ERR_UNSUPPORTED),
    (dict(BS=8), tq.TQ_ERR_UNSUPPORTED),
    (dict(head_dim=64), tq.TQ_ERR_UNSUPPORTED),
    (dict(S=0), tq.TQ_ERR_SHAPE),
    (dict(maxlen=257), tq.TQ_ERR_COVERAGE),
    (dict(MB=1, maxlen=17, P=1), tq.TQ_ERR_COVERAGE),
    (dict(scale=0.0), tq.TQ_ERR_SCALE),
    (dict(cache=A + 8), tq.TQ_ERR_MISALIGNED),
    (dict(cent=A + 2), tq.TQ_ERR_MISALIGNED),
])
def test_tq4_rejects(lib, fused, kw, status):
    """The 4-bit entry points check their arguments on the host before any launch."""
    assert call_tq4(lib, fused=fused, **kw) == status


def test_tq4_block_bytes():
    assert tq.tq4_block_bytes(8, 32) == 8 * 32 * 128 + 8 * 3 * 32 * 2
    assert tq.tq4_block_bytes(1, 16) == 16 * 134
    assert tq.tq4_block_bytes(2, 8) == 0
    assert tq.tq4_block_bytes(0, 16) == 0


def call_reduce(lib, *, part=None, sl=A, out=A, QG=8, Hkv=2, G=1, S=2, P=1, maxlen=64):
    ps = tq.PartialsStruct(*(part or (A, A, A)))
    ext = tq.Extent(S, 1, 1, P, maxlen, 128)
    return lib.tq_decode_reduce(ctypes.byref(ps), sl, out, Hkv, QG, G, ctypes.byref(ext), None)


@pytest.mark.parametrize("kw,status", [
    (dict(sl=0), tq.TQ_ERR_NULL),
    (dict(out=0), tq.TQ_ERR_NULL),
    (dict(part=(0, A, A)), tq.TQ_ERR_NULL),
    (dict(QG=5), tq.TQ_ERR_UNSUPPORTED),
    (dict(S=0), tq.TQ_ERR_SHAPE),
    (dict(P=0), tq.TQ_ERR_SHAPE),
    (dict(G=0), tq.TQ_ERR_SHAPE),
    (dict(maxlen=257), tq.TQ_ERR_COVERAGE),
    (dict(out=A + 8), tq.TQ_ERR_MISALIGNED),
    (dict(part=(A, A + 2, A)), tq.TQ_ERR_MISALIGNED),
])
def test_reduce_rejects(lib, kw, status):
    assert call_reduce(lib, **kw) == status


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 1, 16, 128), dtype=torch.uint8)
    sc = torch.zeros((1, 1, 2, 16))
    bt = torch.zeros((1, 1), dtype=torch.int32)
    sl = torch.ones((1,), dtype=torch.int32)
    with pytest.raises(TypeError):
        tq.decode(q, k, k, sc, bt, sl, max_seq_len=1)


def test_product_path_does_not_import_the_oracle():
    """The library's Python package and sources never reference the oracle."""
    pkg = os.path.join(ROOT, "paged_gqa_decode_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle.c" not in text and "liboracle" not in text, f


def call_kv_write(lib, *, ptrs=None, T=4, Hkv=2, BS=16, NB=8, D=128, layout=0):
    ptrs = ptrs or [A] * 6
    return lib.tq_kv_write(*ptrs, T, Hkv, BS, NB, D, layout, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), tq.TQ_ERR_SHAPE),
    (dict(Hkv=0), tq.TQ_ERR_SHAPE),
    (dict(NB=0), tq.TQ_ERR_SHAPE),
    (dict(NB=1 << 30, BS=32), tq.TQ_ERR_SHAPE),
    (dict(BS=8), tq.TQ_ERR_UNSUPPORTED),
    (dict(D=64), tq.TQ_ERR_UNSUPPORTED),
    (dict(layout=2), tq.TQ_ERR_UNSUPPORTED),
    (dict(layout=-1), tq.TQ_ERR_UNSUPPORTED),
    (dict(ptrs=[A, A, 0, A, A, A]), tq.TQ_ERR_NULL),
    (dict(ptrs=[A + 4, A, A, A, A, A]), tq.TQ_ERR_MISALIGNED),
    (dict(ptrs=[A, A, A, A, A, A + 8]), tq.TQ_ERR_MISALIGNED),
    (dict(ptrs=[A, A, A + 2, A, A, A]), tq.TQ_ERR_MISALIGNED),
])
def test_kv_write_rejects(lib, kw, status):
    assert call_kv_write(lib, **kw) == status


def test_kv_write_zero_tokens_is_a_noop(lib):
    assert call_kv_write(lib, ptrs=[0] * 6, T=0) == tq.TQ_OK


def _fp8_args(S=2, Hkv=2, QG=8, BS=16, NB=4, mb=3):
    import torch
    return dict(q=torch.zeros((S, Hkv * QG, 128), dtype=torch.bfloat16),
                k_cache=torch.zeros((NB, Hkv, BS, 128), dtype=torch.uint8),
                v_cache=torch.zeros((NB, Hkv, BS, 128), dtype=torch.uint8),
                kv_scales=torch.zeros((NB, Hkv, 2, BS), dtype=torch.float32),
                block_tables=torch.zeros((S, mb), dtype=torch.int32),
                seq_lens=torch.ones((S,), dtype=torch.int32))


@pytest.mark.parametrize("field,bad,err", [
    ("q", lambda a: a["q"].float(), TypeError),
    ("q", lambda a: a["q"][:, :12].contiguous(), ValueError),
    ("k_cache", lambda a: a["k_cache"].to(__import__("torch").int8), TypeError),
    ("v_cache", lambda a: a["v_cache"][:, :, :8].contiguous(), ValueError),
    ("kv_scales", lambda a: a["kv_scales"].double(), TypeError),
    ("kv_scales", lambda a: a["kv_scales"][:, :1].contiguous(), ValueError),
    ("block_tables", lambda a: a["block_tables"].long(), TypeError),
    ("block_tables", lambda a: a["block_tables"][:1].contiguous(), ValueError),
    ("seq_lens", lambda a: a["seq_lens"].long(), TypeError),
    ("seq_lens", lambda a: a["seq_lens"][:1].contiguous(), ValueError),
])
@pytest.mark.parametrize("entry", ["tq_decode", "tq_decode_fused"])
def test_binding_refuses_wrong_layouts(entry, field, bad, err):
    """A tensor of the wrong dtype or shape is refused before any pointer reaches the
    library (checked ahead of the device, so CPU tensors show it)."""
    import torch
    a = _fp8_args()
    a[field] = bad(a)
    common = (2, 8, 16, 1, 0.1)
    kw = dict(num_partitions=1, max_seq_len=1)
    with pytest.raises(err, match=field):
        if entry == "tq_decode":
            part = tq.Partials(out=torch.zeros((2, 2, 1, 8, 128)), max_logits=torch.zeros((2, 2, 1, 8)),
                               exp_sums=torch.zeros((2, 2, 1, 8)))
            tq.tq_decode(*a.values(), part, *common, **kw)
        else:
            out = torch.zeros((2, 16, 128), dtype=torch.bfloat16)
            tq.tq_decode_fused(*a.values(), out, *common, **kw)


def test_binding_refuses_wrong_partials_and_pool():
    import torch
    a = _fp8_args()
    good = dict(out=torch.zeros((2, 2, 3, 8, 128)), max_logits=torch.zeros((2, 2, 3, 8)),
                exp_sums=torch.zeros((2, 2, 3, 8)))
    for name, t in (("out", torch.zeros((2, 2, 2, 8, 128))), ("max_logits", torch.zeros((2, 2, 3, 6))),
                    ("exp_sums", torch.zeros((2, 2, 3, 8), dtype=torch.float16))):
        part = tq.Partials(**{**good, name: t})
        with pytest.raises((TypeError, ValueError), match=f"partials.{name}"):
            tq.tq_decode(*a.values(), part, 2, 8, 16, 1, 0.1, num_partitions=3, max_seq_len=1)
        with pytest.raises((TypeError, ValueError), match=f"partials.{name}"):
            tq.tq_decode_reduce(part, a["seq_lens"], torch.zeros((2, 16, 128), dtype=torch.bfloat16),
                                2, 8, 1, num_partitions=3, max_seq_len=1)
    with pytest.raises(ValueError, match="num_blocks"):
        tq.tq_decode(*a.values(), tq.Partials(**good), 2, 8, 16, 1, 0.1, num_partitions=3,
                     max_seq_len=1, num_blocks=5)
    with pytest.raises(TypeError, match="out"):
        tq.tq_decode_reduce(tq.Partials(**good), a["seq_lens"], torch.zeros((2, 16, 128)),
                            2, 8, 1, num_partitions=3, max_seq_len=1)


def test_binding_refuses_wrong_tq4_and_writer_layouts():
    import torch
    S, Hkv, QG, BS = 2, 2, 8, 16
    bb = tq.tq4_block_bytes(Hkv, BS)
    q = torch.zeros((S, Hkv * QG, 128), dtype=torch.bfloat16)
    bt = torch.zeros((S, 3), dtype=torch.int32)
    sl = torch.ones((S,), dtype=torch.int32)
    out = torch.zeros((S, Hkv * QG, 128), dtype=torch.bfloat16)
    cent = torch.zeros((16,), dtype=torch.float32)
    with pytest.raises(ValueError, match="kv_cache"):
        tq.tq4_decode_fused(q, torch.zeros((4, bb - 1), dtype=torch.uint8), cent, bt, sl, out, Hkv, QG,
                            BS, 1, 0.1, num_partitions=1, max_seq_len=1)
    with pytest.raises(ValueError, match="centroids"):
        tq.tq4_decode_fused(q, torch.zeros((4, bb), dtype=torch.uint8), cent[:8].contiguous(), bt, sl,
                            out, Hkv, QG, BS, 1, 0.1, num_partitions=1, max_seq_len=1)
    k = torch.zeros((4, Hkv, BS, 128), dtype=torch.uint8)
    sc = torch.zeros((4, Hkv, 2, BS), dtype=torch.float32)
    rows = torch.zeros((5, Hkv, 128), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="slot_mapping"):
        tq.tq_kv_write(rows, rows, torch.zeros((5,), dtype=torch.int64), k, k, sc)
    with pytest.raises(ValueError, match="kv_scales"):
        tq.tq_kv_write(rows, rows, torch.zeros((5,), dtype=torch.int32), k, k, sc[:, :, :1].contiguous())
    with pytest.raises(TypeError, match="v_new"):
        tq.tq_kv_write(rows, rows.float(), torch.zeros((5,), dtype=torch.int32), k, k, sc)


def test_static_entry_point_rejects_before_touching_the_device(lib):
    """tq_decode_fused_static: the argument checks of tq_decode_fused, then TQ_ERR_SCRATCH for a
    batch whose counters (4 B per (s, h)) pass the static scratch's 1 MiB counter region; none
    of these calls reaches the device."""
    assert tq.STATIC_SCRATCH_BYTES == 8 << 20 and tq.STATIC_COUNTER_BYTES == 1 << 20

    def call(S, Hkv, ptrs=None, QG=8, scale=0.088, maxlen=64):
        ext = tq.Extent(S, 8, 4, 1, maxlen, 128)
        return lib.tq_decode_fused_static(*(ptrs or [A] * 7), Hkv, QG, 16, 1, scale,
                                          ctypes.byref(ext), None)

    assert call(2, 2, ptrs=[A] * 6 + [0]) == tq.TQ_ERR_NULL
    assert call(2, 2, QG=7) == tq.TQ_ERR_UNSUPPORTED
    assert call(2, 2, scale=0.0) == tq.TQ_ERR_SCALE
    assert call(1024, 257) == tq.TQ_ERR_SCRATCH      # 263168 (s, h) counters > 1 MiB
    assert call(2048, 129) == tq.TQ_ERR_SCRATCH      # the per-(s, h) plan, same bound
