"""C-ABI checks that need no GPU: the library loads, exports every function
include/paged_gqa.h declares, and rejects invalid arguments with the
documented status codes before anything is launched (argument checks never
dereference device pointers, so host placeholders stand in for them)."""
import ctypes
import os
import re

import pytest

import paged_gqa_attention_hd256_amd as pga
from paged_gqa_attention_hd256_amd import _KV

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_gqa.h")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EWS, ESCRATCH = 0, 1, 2, 3, 4, 5, 8


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pga.library_path()):
        from paged_gqa_attention_hd256_amd import build
        build.build(verbose=False)
    return pga.load_library()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"paged_attn_verify", "paged_attn_prefill_prefix", "sparse_paged_attn"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pga_abi_version() == 4


def test_status_strings(lib):
    for code in range(0, 9):
        assert pga.status_string(code) != "unknown status"
    assert pga.status_string(99) == "unknown status"


# Host buffers stand in for device memory: validation never dereferences them.
_buf = ctypes.create_string_buffer(1 << 16)
_base = (ctypes.addressof(_buf) + 255) & ~255


def P(off=0):
    return _base + off


def kv_struct(**over):
    s = _KV()
    s.k_cache, s.v_cache = P(0), P(4096)
    s.dtype, s.num_kv_heads, s.head_dim, s.page_size, s.num_pages = 2, 1, 256, 16, 128
    s.k_stride_page, s.k_stride_token, s.k_stride_head = 16 * 256, 256, 256
    s.v_stride_page, s.v_stride_token, s.v_stride_head = 16 * 256, 256, 256
    s.block_table, s.block_table_stride = P(8192), 64
    s.k_descale = s.v_descale = None
    for k, v in over.items():
        setattr(s, k, v)
    return s


def verify(lib, kv=None, **kw):
    a = dict(q=P(), q_dtype=1, qds=None, hq=16, nseq=2, cuq=P(16384), lk=P(16384 + 64), maxq=4, maxk=1000,
             scale=0.0625, split=0, ws=None, wsb=0, out=P(20000), lse=None)
    a.update(kw)
    kv = kv or kv_struct()
    return lib.paged_attn_verify(a["q"], a["q_dtype"], a["qds"], a["hq"], a["nseq"], a["cuq"], a["lk"], a["maxq"],
                                 a["maxk"], ctypes.byref(kv), a["scale"], a["split"], a["ws"], a["wsb"], a["out"],
                                 a["lse"], None)


def test_verify_rejects_invalid_arguments(lib):
    assert verify(lib, q=None) == ENULL
    assert verify(lib, out=None) == ENULL
    assert verify(lib, kv=kv_struct(block_table=None)) == ENULL
    assert verify(lib, q_dtype=2) == EDTYPE
    assert verify(lib, kv=kv_struct(dtype=7)) == EDTYPE
    assert verify(lib, kv=kv_struct(head_dim=128)) == ESHAPE
    assert verify(lib, kv=kv_struct(num_kv_heads=2), hq=15) == ESHAPE
    assert verify(lib, maxq=0) == ESHAPE
    assert verify(lib, maxq=5) == ESHAPE
    assert verify(lib, hq=32) == EUNSUP                     # 32 x 4 rows > 64
    assert verify(lib, nseq=-1) == ESHAPE
    assert verify(lib, maxk=-1) == ESHAPE
    assert verify(lib, split=100) == ESHAPE                 # not a multiple of 64
    assert verify(lib, kv=kv_struct(page_size=24)) == EUNSUP
    assert verify(lib, kv=kv_struct(page_size=8)) == EUNSUP
    assert verify(lib, kv=kv_struct(k_stride_token=250)) == EUNSUP
    assert verify(lib, kv=kv_struct(k_cache=P(8))) == EUNSUP   # misaligned pool
    assert verify(lib, q=P(4)) == EUNSUP
    assert verify(lib, kv=kv_struct(block_table_stride=10)) == ESHAPE  # < ceil(1000 / 16)
    assert verify(lib, scale=float("nan")) == ESHAPE
    need = pga.verify_workspace_bytes(16, 1, 2, 4, 1000, 0)
    assert need > 0
    assert verify(lib, ws=None, wsb=0) == EWS
    assert verify(lib, ws=P(), wsb=need - 1) == EWS


def test_verify_rejects_plans_past_int32_positions(lib):
    # The kernels index the flattened tile list and the workspace slots with
    # int32 positions: a batch whose list would not fit is refused before any
    # launch (no workspace is looked at), and the workspace query returns 0.
    big = dict(nseq=1 << 20, maxk=1 << 20)                  # 2^20 units x 16,384 tiles
    assert verify(lib, kv=kv_struct(block_table_stride=1 << 16), **big, ws=P(), wsb=1 << 62) == EUNSUP
    assert pga.verify_workspace_bytes(16, 1, 1 << 20, 4, 1 << 20, 0) == 0
    assert pga.verify_workspace_bytes(16, 1, 1 << 20, 4, 1 << 20, 64) == 0
    # just inside: 2^15 sequences x 16,384 tiles + 3 start positions < 2^30
    assert pga.verify_workspace_bytes(16, 1, 1 << 15, 4, 1 << 20, 0) > 0


def verify_noalloc(lib, kv=None, **kw):
    a = dict(q=P(), q_dtype=1, qds=None, hq=16, nseq=2, cuq=P(16384), lk=P(16384 + 64), maxq=4, maxk=1000,
             scale=0.0625, split=0, out=P(20000), lse=None)
    a.update(kw)
    kv = kv or kv_struct()
    return lib.paged_attn_verify_noalloc(a["q"], a["q_dtype"], a["qds"], a["hq"], a["nseq"], a["cuq"], a["lk"],
                                         a["maxq"], a["maxk"], ctypes.byref(kv), a["scale"], a["split"], a["out"],
                                         a["lse"], None)


def test_verify_noalloc_checks_before_touching_the_scratch(lib):
    # Argument checks are those of paged_attn_verify ...
    assert verify_noalloc(lib, q=None) == ENULL
    assert verify_noalloc(lib, q_dtype=2) == EDTYPE
    assert verify_noalloc(lib, maxq=5) == ESHAPE
    assert verify_noalloc(lib, hq=32) == EUNSUP
    assert verify_noalloc(lib, nseq=0) == OK          # nothing to do: no scratch lookup, no launch
    # ... and bounds whose partials exceed the fixed scratch are refused
    # before its device address is looked up: 4,096 sequences x 1,024
    # segments of 64 keys x 64 rows x 256 fp16 values is far past 128 MiB.
    big = dict(nseq=4096, maxk=65536, split=64)
    assert verify_noalloc(lib, kv=kv_struct(block_table_stride=4096), **big) == ESCRATCH


def test_verify_nothing_to_do_returns_ok_without_launch(lib):
    assert verify(lib, nseq=0) == OK
    assert verify(lib, maxk=0) == OK


def _ws_expect(hq, hkv, nseq, maxq, maxk, split):
    # One slot of r * max_q_len rows x (256 + 1) fp32 values per (segment,
    # workgroup) piece -- at most #segments + #workgroups of them.
    tiles = -(-maxk // 64)
    seg_tiles = split // 64 if split else max(1, tiles)
    segs = max(1, -(-tiles // seg_tiles))
    units = nseq * hkv
    # runs of at least 1 position over the list of tiles plus 5 start
    # positions per segment, capped at 1024 workgroups
    wg_cap = min(1024, max(1, units * (tiles + 5 * segs)))
    slots = units * segs + wg_cap
    rows = hq // hkv * maxq
    o = slots * rows * 256 * 4
    lse = (slots * rows * 4 + 15) & ~15
    return ((o + 255) & ~255) + lse + (units * 2 + 4) * 4  # then the per-unit plan and tiles per workgroup


def test_verify_workspace_plan(lib):
    for args in [(16, 1, 64, 4, 32768, 0), (32, 2, 128, 3, 65536, 4096), (16, 1, 2, 2, 1000, 0),
                 (16, 1, 64, 4, 4096, 1 << 20), (8, 1, 3, 4, 64, 64)]:
        assert pga.verify_workspace_bytes(*args) == _ws_expect(*args), args
    assert pga.verify_split_tokens(16, 1, 64, 4, 32768, 0) == 32768      # auto: whole history per segment
    assert pga.verify_split_tokens(32, 2, 128, 3, 65536, 4096) == 4096
    assert pga.verify_workspace_bytes(16, 1, 2, 4, 1000, 100) == 0       # invalid split -> 0
    assert pga.verify_workspace_bytes(16, 1, 0, 4, 1000, 0) == 0         # no sequences


def prefill(lib, kv=None, **kw):
    a = dict(q=P(), q_dtype=2, qds=None, hq=8, nseq=1, cuq=P(16384), cuk=P(16384 + 64), maxq=100, maxk=300,
             scale=0.0625, out=P(20000), lse=None)
    a.update(kw)
    kv = kv or kv_struct()
    return lib.paged_attn_prefill_prefix(a["q"], a["q_dtype"], a["qds"], a["hq"], a["nseq"], a["cuq"], a["cuk"],
                                         a["maxq"], a["maxk"], ctypes.byref(kv), a["scale"], a["out"], a["lse"], None)


def test_prefill_rejects_invalid_arguments(lib):
    assert prefill(lib, cuk=None) == ENULL
    assert prefill(lib, q_dtype=3) == EDTYPE
    assert prefill(lib, kv=kv_struct(dtype=1)) == EDTYPE      # FP8 Q needs FP8 KV
    assert prefill(lib, hq=128) == EUNSUP                     # 128 query heads per kv head
    assert prefill(lib, maxq=-1) == ESHAPE
    assert prefill(lib, kv=kv_struct(block_table_stride=5)) == ESHAPE
    assert prefill(lib, nseq=0) == OK
    assert prefill(lib, maxq=0) == OK


def sparse(lib, kv=None, **kw):
    a = dict(q=P(), q_dtype=1, qds=None, hq=24, ntok=8, nseq=1, cuq=P(16384), lk=P(16384 + 64), idx=P(30000),
             stride=64, nsel=64, scale=0.0625, ws=None, wsb=0, out=P(20000), lse=None)
    a.update(kw)
    kv = kv or kv_struct(num_kv_heads=2)
    return lib.sparse_paged_attn(a["q"], a["q_dtype"], a["qds"], a["hq"], a["ntok"], a["nseq"], a["cuq"], a["lk"],
                                 a["idx"], a["stride"], a["nsel"], ctypes.byref(kv), a["scale"], a["ws"], a["wsb"],
                                 a["out"], a["lse"], None)


def test_sparse_rejects_invalid_arguments(lib):
    assert sparse(lib, idx=None) == ENULL
    assert sparse(lib, q_dtype=2) == EDTYPE
    assert sparse(lib, stride=10) == ESHAPE                   # fewer columns than num_selected
    assert sparse(lib, nsel=-1) == ESHAPE
    assert sparse(lib, nseq=0) == ESHAPE                      # rows without a sequence
    assert sparse(lib, hq=25) == ESHAPE
    assert sparse(lib, kv=kv_struct(num_kv_heads=2, num_pages=1 << 30, page_size=64)) == EUNSUP
    assert sparse(lib, ntok=0) == OK
    # 8 rows x 2 kv heads leave the GPU idle: the lists are cut into pieces,
    # which need a workspace of the reported size and alignment.
    assert sparse(lib, nsel=2048, stride=2048, ws=P(1 << 20), wsb=16) == EWS
    assert sparse(lib, nsel=2048, stride=2048, ws=P((1 << 20) + 4), wsb=1 << 40) == EUNSUP


def test_sparse_split_plan(lib):
    def cdiv(a, b):
        return -(-a // b)

    def expect(hq, hkv, ntok, nsel):
        # The piece count with the fewest rounds x piece tiles on a 256-CU part
        # (2,048 FP8 and 1,024 BF16 waves per round; 3 tiles to start a piece).
        jobs = ntok * hkv * cdiv(hq // hkv, 16)

        def piece_len(s):
            return max(32, cdiv(cdiv(nsel, s), 32) * 32)

        length = piece_len(1)
        if 0 < jobs < 4096 and nsel > 0:
            costs = []
            for s in range(1, max(1, min(32, cdiv(nsel, 256))) + 1):
                ln = piece_len(s)
                pieces = cdiv(nsel, ln)
                rounds = cdiv(jobs * pieces, 2048) + cdiv(jobs * pieces, 1024)
                costs.append((rounds * (cdiv(ln, 16) + 3), s, ln))
            length = min(costs)[2]
        splits = cdiv(nsel, length) if nsel > 0 else 1
        ws = 0
        if splits > 1:
            slots = ntok * hq * splits
            ws = ((slots * 256 * 4 + 255) & ~255) + slots * 4
        return splits, ws

    for args in [(24, 2, 8, 2048), (24, 2, 8192, 2051), (24, 2, 260, 2051), (12, 1, 3, 100), (32, 1, 1, 5000),
                 (24, 2, 0, 2051), (24, 2, 10, 0)]:
        splits, ws = expect(*args)
        assert lib.sparse_paged_attn_splits(*args) == splits, args
        assert lib.sparse_paged_attn_workspace_bytes(*args) == ws, args
    assert lib.sparse_paged_attn_splits(24, 2, 8, 2048) == 8
    assert lib.sparse_paged_attn_splits(24, 2, 8192, 2051) == 1      # the large-row workload: no split
    # 260 rows: 7 pieces (455 FP8 workgroups, two rounds of 256 CUs) rather
    # than 8 (520 workgroups: a third round for 8 of them).
    assert lib.sparse_paged_attn_splits(24, 2, 260, 2051) == 7
    assert lib.sparse_paged_attn_splits(25, 2, 8, 64) == 0          # invalid head counts


def quantize(lib, kv=None, **kw):
    a = dict(q=P(), hq=8, ntok=16, qds=None, qfp8=P(20000), qds_out=P(40000), k_new=P(24576), v_new=P(28672),
             nseq=1, cuq=P(16384), cuk=P(16384 + 64), ws=P(1 << 15), wsb=4096 + 128 * 1024 + 256)
    a.update(kw)
    kv = kv or kv_struct()
    return lib.prefill_quantize_fp8(a["q"], a["hq"], a["ntok"], a["qds"], a["qfp8"], a["qds_out"], a["k_new"],
                                    a["v_new"], a["nseq"], a["cuq"], a["cuk"], ctypes.addressof(kv), a["ws"],
                                    a["wsb"], None)


def test_quantize_rejects_invalid_arguments(lib):
    # 1024 per-workgroup maxima, then 1024 barrier slots of 128 bytes and a flag block
    assert lib.prefill_quantize_fp8_workspace_bytes() == 4096 + 128 * 1024 + 256
    assert quantize(lib, q=None) == ENULL
    assert quantize(lib, qfp8=None) == ENULL
    assert quantize(lib, qds_out=None) == ENULL                # the dynamic descale needs somewhere to go
    assert quantize(lib, v_new=None) == ENULL                 # keys without values
    assert quantize(lib, cuk=None) == ENULL
    assert quantize(lib, hq=0) == ESHAPE
    assert quantize(lib, ntok=-1) == ESHAPE
    assert quantize(lib, nseq=0) == ESHAPE                    # new tokens without a sequence
    assert quantize(lib, kv=kv_struct(num_kv_heads=5)) == ESHAPE
    assert quantize(lib, kv=kv_struct(dtype=1)) == EDTYPE     # the pool must be FP8
    assert quantize(lib, q=P(8)) == EUNSUP                    # q not 16-byte aligned
    assert quantize(lib, k_new=P(24584)) == EUNSUP
    assert quantize(lib, wsb=4096 + 128 * 1024 + 255) == EWS
    assert quantize(lib, ws=None) == EWS
    assert quantize(lib, ws=P((1 << 15) + 16)) == EUNSUP      # workspace not 256-byte aligned


def validate(lib, kv=None, **kw):
    a = dict(nseq=2, ntok=8, cuq=P(16384), lk=P(16384 + 64), cuk=None, maxq=0, maxk=0, idx=None, stride=0, nsel=0,
             counts=P(40000), host=None)
    a.update(kw)
    kv = kv or kv_struct()
    return lib.pga_validate_inputs(a["nseq"], a["ntok"], a["cuq"], a["lk"], a["cuk"], a["maxq"], a["maxk"],
                                   ctypes.byref(kv), a["idx"], a["stride"], a["nsel"], a["counts"], a["host"], None)


def test_validate_rejects_invalid_host_arguments(lib):
    assert validate(lib, cuq=None) == ENULL
    assert validate(lib, lk=None) == ENULL                     # neither seq_lens_k nor cu_seqlens_k
    assert validate(lib, cuk=P(16384 + 128)) == ENULL          # both
    assert validate(lib, counts=None) == ENULL
    assert validate(lib, nseq=-1) == ESHAPE
    assert validate(lib, kv=kv_struct(page_size=24)) == ESHAPE
    assert validate(lib, idx=P(30000), ntok=-1, stride=8, nsel=8) == ESHAPE
    assert validate(lib, idx=P(30000), stride=4, nsel=8) == ESHAPE
    assert validate(lib, counts=P(40002)) == EUNSUP


def gather(lib, kv=None, **kw):
    a = dict(ntok=8, nseq=1, cuq=P(16384), lk=P(16384 + 64), idx=P(30000), stride=64, nsel=64, out=P(20480))
    a.update(kw)
    kv = kv or kv_struct()
    return lib.sparse_gather_sum(a["ntok"], a["nseq"], a["cuq"], a["lk"], a["idx"], a["stride"], a["nsel"],
                                 ctypes.byref(kv), a["out"], None)


def test_gather_rejects_pools_its_offsets_cannot_address(lib):
    assert gather(lib, ntok=0) == OK
    assert gather(lib, out=None) == ENULL
    # Not evenly spaced: the page stride is not page_size token strides.
    assert gather(lib, kv=kv_struct(k_stride_page=16 * 256 + 256)) == EUNSUP
    # More than 2^24 token rows, a token stride of 2^24 bytes, rows past 4 GiB.
    assert gather(lib, kv=kv_struct(num_pages=(1 << 20) + 1)) == EUNSUP
    assert gather(lib, kv=kv_struct(k_stride_token=1 << 24, k_stride_page=16 << 24)) == EUNSUP
    assert gather(lib, kv=kv_struct(num_pages=1 << 20, k_stride_token=1 << 13, k_stride_page=16 << 13)) == EUNSUP


def verify_gather(lib, kv=None, **kw):
    a = dict(nseq=2, cuq=P(16384), lk=P(16384 + 64), maxq=4, maxk=1000, split=0, out=P(20480))
    a.update(kw)
    kv = kv or kv_struct()
    return lib.paged_attn_verify_gather_sum(a["nseq"], a["cuq"], a["lk"], a["maxq"], a["maxk"], ctypes.byref(kv),
                                            a["split"], a["out"], None)


def test_verify_gather_rejects_invalid_arguments(lib):
    assert verify_gather(lib, nseq=0) == OK
    assert verify_gather(lib, out=None) == ENULL
    assert verify_gather(lib, cuq=None) == ENULL
    assert verify_gather(lib, maxq=5) == ESHAPE
    assert verify_gather(lib, split=10) == ESHAPE
    assert verify_gather(lib, out=P(20481)) == EUNSUP
    assert verify_gather(lib, kv=kv_struct(block_table_stride=10)) == ESHAPE  # fewer columns than the bound's pages
