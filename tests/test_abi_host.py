"""Host-side checks of the C ABI that need no GPU: the library loads and
exports every declared symbol, the split heuristic follows the pages' rules
where the grid fits on the GPU at once and its measured MI355X rule beyond, and invalid arguments come back as status codes before anything is
launched.  Every call here either is host-only (the heuristic, the workspace
size, status names) or fails validation, so no kernel is ever enqueued."""
import ctypes as C
import re
from pathlib import Path

import pytest

import decode_attention_attn_amd as fd

HEADER = Path(__file__).resolve().parents[1] / "include" / "fd_decode_attn.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)   # declarations, not comments
    return sorted(set(re.findall(r"\b(fd_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) >= {"fd_decode_attn_partial", "fd_decode_attn_combine", "fd_decode_attn_paged",
                          "fd_split_heuristic", "fd_workspace_bytes", "fd_status_string"}
    L = fd.lib()
    for n in names:
        assert hasattr(L, n), n


def test_header_constants_match_the_binding():
    text = HEADER.read_text()

    def define(name):
        expr = re.search(rf"#define {name} (.+)", text).group(1)
        expr = re.sub(r"(\d+)u\b", r"\1", expr)
        assert re.fullmatch(r"[\d\s()*<+]+", expr), expr     # integers, *, << only
        return eval(expr)

    assert define("FD_TICKET_BYTES") == fd.TICKET_BYTES
    assert define("FD_MAX_Q_LEN") == fd.MAX_Q_LEN
    assert define("FD_NOALLOC_SCRATCH_BYTES") == fd.NOALLOC_SCRATCH_BYTES


def test_status_strings():
    assert fd.fd_status_string(fd.FD_OK) == "FD_OK"
    assert fd.fd_status_string(fd.FD_ERR_WORKSPACE_TOO_SMALL) == "FD_ERR_WORKSPACE_TOO_SMALL"
    assert fd.fd_status_string(99) == "FD_UNKNOWN_STATUS"


def test_desc_struct_matches_header_field_order():
    text = HEADER.read_text()
    body = re.search(r"typedef struct fd_decode_desc \{(.*?)\} fd_decode_desc;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        names = decl.split(None, 1)[1]
        fields += [re.sub(r"^.*?\**\s*(\w+)$", r"\1", n.strip().split()[-1]) for n in names.split(",")]
    assert fields == [f[0] for f in fd.fd_decode_desc._fields_]


# ----------------------------------------------------------------------------
# split heuristic: the Flash-Decoding page's granularity while the grid fits
# on the GPU at once, larger splits (fewer partials) once it does not
# ----------------------------------------------------------------------------
MI355X_CUS = 256


@pytest.mark.parametrize("B,Hq,Hkv,N,page,split,S", [
    (1, 8, 8, 512, 0, 128, 4),          # tiny MHA
    (1, 32, 32, 4096, 0, 256, 16),      # Llama2-7B-shaped MHA
    (1, 32, 8, 32768, 0, 256, 128),     # long-context GQA
    (4, 64, 8, 131072, 0, 1024, 128),   # unified-max stress shape: 4096 workgroups at split 1024
])
def test_heuristic_reproduces_the_workload_split_sizes(B, Hq, Hkv, N, page, split, S):
    assert fd.fd_split_heuristic(B, Hq, Hkv, N, page, MI355X_CUS) == (split, S)


def test_heuristic_grows_the_split_when_the_grid_is_several_waves():
    # B * Hkv = 512 units, 64 splits of 256 each: 32768 workgroups.  The page
    # would not split at all (512 >= 2 * CUs); here the split grows to the
    # 1024-token cap, still 8192 workgroups at the longest length
    assert fd.fd_split_heuristic(64, 64, 8, 16384, 16, MI355X_CUS) == (1024, 16)
    # a batch that fills the GPU with short requests: one split per request
    assert fd.fd_split_heuristic(256, 64, 8, 512, 16, MI355X_CUS) == (512, 1)
    # between the two: the split that leaves ~8 workgroups per CU
    split, S = fd.fd_split_heuristic(16, 64, 8, 8192, 16, MI355X_CUS)
    assert split == 512 and S == 16 and 16 * 8 * S == 8 * MI355X_CUS
    # a very long request: the split rises so that S stays within 4096
    split, S = fd.fd_split_heuristic(1, 8, 1, 1 << 23, 0, MI355X_CUS)
    assert (split, S) == (2048, 4096)


def test_heuristic_page_example_split_count(golden):
    g = golden("flashdecoding_split_sizes.json")["split_count_example"]
    # the page's example: N = 32768, split 256 -> S = 128; with 16 query heads
    # at B = 1 that is 2048 blocks (one per query head); here a block covers a
    # KV head, so use Hq = Hkv = 16.  2048 workgroups fit on MI355X at once.
    split, S = fd.fd_split_heuristic(g["B"], g["query_heads"], g["query_heads"], g["N"], 0, MI355X_CUS)
    assert split == g["split"] and S == g["S"]
    assert g["B"] * g["query_heads"] * S == g["blocks"]


@pytest.mark.parametrize("page", [1, 16, 32])
def test_heuristic_is_page_aligned_clamped_and_monotone(golden, page):
    gran = golden("flashdecoding_split_sizes.json")["split_granularity"]
    last_S = 0
    for N in [1, 100, 1000, 4096, 10000, 32768, 100000, 131072, 1 << 20]:
        split, S = fd.fd_split_heuristic(1, 32, 8, N, page, MI355X_CUS)
        assert split % page == 0
        assert S == -(-N // split)
        assert S >= last_S
        last_S = S
        if 8 * -(-N // 256) <= 8 * MI355X_CUS:            # the grid fits at once: the page's range
            assert gran["lo"] <= split <= gran["hi"]
        else:                                            # several waves: ~8 workgroups per CU
            assert 256 <= split <= 1024 + page
            assert 8 * S >= 0.9 * 8 * MI355X_CUS or split >= 1024   # (page rounding)


def test_heuristic_rejects_bad_arguments():
    for args in [(0, 8, 8, 100, 0, 256), (1, 8, 3, 100, 0, 256), (1, 8, 8, -1, 0, 256),
                 (1, 8, 8, 100, -16, 256), (1, 8, 8, 100, 0, 0)]:
        with pytest.raises(fd.FdError) as e:
            fd.fd_split_heuristic(*args)
        assert e.value.status == fd.FD_ERR_INVALID_ARG


# ----------------------------------------------------------------------------
# workspace layout
# ----------------------------------------------------------------------------
def test_workspace_bytes_layout(golden):
    d = fd.make_desc(1, 32, 8, 128, "bf16", split_size=256, max_splits=128)
    rows = 1 * 32 * 128
    r256 = lambda x: (x + 255) // 256 * 256
    assert fd.fd_workspace_bytes(d) == fd.TICKET_BYTES + r256(rows * 128 * 4) + 2 * r256(rows * 4)
    # the page's intermediate-buffer example counts 16-bit O; ours is fp32, twice it
    g = golden("flashdecoding_split_sizes.json")["intermediate_buffer_example"]
    assert g["B"] * g["H"] * g["S"] * g["d"] * g["elem_bytes"] == g["bytes"]
    assert r256(rows * 128 * 4) == 2 * g["bytes"]


def test_workspace_bytes_zero_for_invalid_desc():
    assert fd.fd_workspace_bytes(fd.make_desc(1, 6, 4, 128, "bf16", max_splits=4)) == 0


# ----------------------------------------------------------------------------
# validation (every call below fails before any launch)
# ----------------------------------------------------------------------------
def _partial_status(desc, kv_capacity=16, with_tensors=False):
    L = fd.lib()
    return L.fd_decode_attn_partial(C.byref(desc), None, None, None, kv_capacity, None, None, None, None,
                                    None, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), fd.FD_ERR_INVALID_ARG),               # Hq not a multiple of Hkv
    (dict(Hq=64, Hkv=2), fd.FD_ERR_UNSUPPORTED),              # group of 32 query heads
    (dict(d=96), fd.FD_ERR_UNSUPPORTED),
    (dict(split_size=0), fd.FD_ERR_INVALID_ARG),
    (dict(split_size=(1 << 20) + 1), fd.FD_ERR_INVALID_ARG),
    (dict(split_size=1 << 20, max_splits=4096), fd.FD_ERR_INVALID_ARG),   # 2^32 tokens
    (dict(split_size=1 << 19, max_splits=4096), fd.FD_ERR_INVALID_ARG),   # 2^31 tokens
    (dict(max_splits=0), fd.FD_ERR_INVALID_ARG),
    (dict(max_splits=4097), fd.FD_ERR_INVALID_ARG),
    (dict(mode="unified", phi=0.0, lo=1.0, hi=-1.0), fd.FD_ERR_INVALID_ARG),   # lo > hi
    (dict(mode="unified", phi=-6.0, lo=-6.0, hi=60.0), fd.FD_ERR_INVALID_ARG),  # hi - phi > 64
    (dict(mode="unified", phi=0.0, lo=-65.0, hi=0.0), fd.FD_ERR_INVALID_ARG),   # phi - lo > 64
    (dict(scale=float("nan")), fd.FD_ERR_INVALID_ARG),
    (dict(), fd.FD_ERR_INVALID_ARG),                            # valid desc, NULL tensors
])
def test_partial_validation(kw, status):
    base = dict(B=1, Hq=8, Hkv=8, d=128, kv_dtype="bf16", split_size=256, max_splits=4)
    base.update(kw)
    B, Hq, Hkv, d, dt = (base.pop(x) for x in ("B", "Hq", "Hkv", "d", "kv_dtype"))
    desc = fd.make_desc(B, Hq, Hkv, d, dt, **base)
    assert _partial_status(desc) == status


def test_partial_rejects_bad_enum_codes_and_negative_capacity():
    desc = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4)
    desc.kv_dtype = 7
    assert _partial_status(desc) == fd.FD_ERR_INVALID_ARG
    desc = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4)
    desc.mode = 5
    assert _partial_status(desc) == fd.FD_ERR_INVALID_ARG
    desc = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4)
    desc.kernel = 9
    assert _partial_status(desc) == fd.FD_ERR_INVALID_ARG
    desc = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4)
    assert _partial_status(desc, kv_capacity=-1) == fd.FD_ERR_INVALID_ARG


def test_fp8_descriptor_validation():
    """8-bit caches need an f16 or bf16 q, finite scales and a 16/32-bit output."""
    ok = fd.make_desc(1, 8, 8, 128, "fp8", max_splits=4, k_scale=0.5, v_scale=2.0)
    assert ok.q_dtype == fd.FD_BF16 and ok.out_dtype == fd.FD_BF16
    assert _partial_status(ok) == fd.FD_ERR_INVALID_ARG          # valid desc, NULL tensors
    bad = fd.make_desc(1, 8, 8, 128, "fp8", max_splits=4, q_dtype="f32")
    assert _partial_status(bad) == fd.FD_ERR_INVALID_ARG
    bad = fd.make_desc(1, 8, 8, 128, "fp8", max_splits=4, k_scale=float("inf"))
    assert _partial_status(bad) == fd.FD_ERR_INVALID_ARG
    bad = fd.make_desc(1, 8, 8, 128, "fp8", max_splits=4, v_scale=float("nan"))
    assert _partial_status(bad) == fd.FD_ERR_INVALID_ARG
    bad = fd.make_desc(1, 8, 8, 128, "fp8", max_splits=4, out_dtype="fp8")
    assert _partial_status(bad) == fd.FD_ERR_INVALID_ARG
    # q_dtype is ignored for 16-bit caches
    other = fd.make_desc(0, 8, 8, 128, "bf16", max_splits=4)
    other.q_dtype = 99
    assert _partial_status(other) == fd.FD_OK
    assert fd.fd_workspace_bytes(ok) == fd.fd_workspace_bytes(fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4))


def test_multi_query_descriptor_validation():
    """Any q_len up to FD_MAX_Q_LEN with q_len * Hq < 2^31 is valid (rows beyond
    a workgroup's go in query tiles; INVALID_ARG below only says validation
    passed: the test hands no tensors)."""
    ok = fd.FD_ERR_INVALID_ARG
    assert _partial_status(fd.make_desc(1, 32, 8, 128, "bf16", max_splits=4, q_len=4)) == ok
    assert _partial_status(fd.make_desc(1, 32, 8, 128, "bf16", max_splits=4, q_len=9)) == ok
    assert _partial_status(fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4, q_len=33)) == ok
    assert _partial_status(fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4, q_len=fd.MAX_Q_LEN)) == ok
    assert _partial_status(fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4,
                                        q_len=fd.MAX_Q_LEN + 1)) == fd.FD_ERR_UNSUPPORTED
    # q_len * Hq = 2^31 query rows per request
    assert _partial_status(fd.make_desc(1, 32768, 2048, 128, "bf16", max_splits=4,
                                        q_len=fd.MAX_Q_LEN)) == fd.FD_ERR_UNSUPPORTED
    assert _partial_status(fd.make_desc(1, 32767 * 16, 32767, 128, "bf16", max_splits=4,
                                        q_len=4096)) == ok
    # requests x query tiles of 16 rows (one token each for a group of 16) <= 65535
    assert _partial_status(fd.make_desc(1023, 16, 1, 64, "bf16", max_splits=4, q_len=64)) == ok
    assert _partial_status(fd.make_desc(1024, 16, 1, 64, "bf16", max_splits=4, q_len=64)) == fd.FD_ERR_UNSUPPORTED
    assert _partial_status(fd.make_desc(1, 8, 1, 64, "bf16", max_splits=4, q_len=65535 * 2)) == fd.FD_ERR_UNSUPPORTED
    assert _partial_status(fd.make_desc(2, 8, 1, 64, "bf16", max_splits=4, q_len=65534)) == ok
    one = fd.make_desc(2, 8, 8, 128, "bf16", max_splits=4)
    zero = fd.make_desc(2, 8, 8, 128, "bf16", max_splits=4, q_len=0)
    four = fd.make_desc(2, 8, 8, 128, "bf16", max_splits=4, q_len=4)
    assert fd.fd_workspace_bytes(zero) == fd.fd_workspace_bytes(one)
    T = fd.TICKET_BYTES
    assert fd.fd_workspace_bytes(four) - T >= 4 * (fd.fd_workspace_bytes(one) - T) - 3 * 256 * 3


def test_empty_batch_is_a_no_op():
    desc = fd.make_desc(0, 8, 8, 128, "bf16", max_splits=4)
    assert _partial_status(desc) == fd.FD_OK
    L = fd.lib()
    assert L.fd_decode_attn_combine(C.byref(desc), None, None, None, None, None, None, None) == fd.FD_OK


def test_paged_validation():
    L = fd.lib()
    desc = fd.make_desc(2, 8, 8, 128, "bf16", split_size=100, max_splits=4)
    # split not a multiple of the page size
    assert L.fd_decode_attn_paged(C.byref(desc), None, None, None, 10, 16, None, 8, None, None, 0, None, None,
                                  None, None, None) == fd.FD_ERR_INVALID_ARG
    desc = fd.make_desc(2, 8, 8, 128, "bf16", split_size=256, max_splits=4)
    assert L.fd_decode_attn_paged(C.byref(desc), None, None, None, 10, 0, None, 8, None, None, 0, None, None,
                                  None, None, None) == fd.FD_ERR_INVALID_ARG
    # NULL tensors
    assert L.fd_decode_attn_paged(C.byref(desc), None, None, None, 10, 16, None, 8, None, None, 0, None, None,
                                  None, None, None) == fd.FD_ERR_INVALID_ARG


def test_combine_validation():
    L = fd.lib()
    desc = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4)
    assert L.fd_decode_attn_combine(C.byref(desc), None, None, None, None, None, None, None) == \
        fd.FD_ERR_INVALID_ARG
    desc.d = 32
    assert L.fd_decode_attn_combine(C.byref(desc), None, None, None, None, None, None, None) == \
        fd.FD_ERR_UNSUPPORTED


# ----------------------------------------------------------------------------
# alignment: q, K, V, part_o and out move 16 bytes at a time; the other
# tensors need their element size.  Each call below hands well-formed fake
# device addresses with exactly one of them misaligned, so validation must
# refuse it before anything is launched.
# ----------------------------------------------------------------------------
_A = 0x7F0000000000          # a 256-byte aligned stand-in address (never dereferenced)


def _addr(i, off=0):
    return C.c_void_p(_A + i * 0x100000 + off)


@pytest.mark.parametrize("pos,off", [(0, 8), (1, 4), (2, 2), (4, 2), (5, 8), (6, 2), (7, 1), (9, 2)])
def test_partial_rejects_misaligned_pointers(pos, off):
    """Positions: 0 q, 1 k, 2 v, 4 seq_lens, 5 part_o, 6 part_m, 7 part_l, 9 fallback_count."""
    L = fd.lib()
    desc = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4)
    args = [_addr(i) for i in range(10)]
    args[3] = C.c_int32(16)
    args[pos] = _addr(pos, off)
    assert L.fd_decode_attn_partial(C.byref(desc), *args, None) == fd.FD_ERR_INVALID_ARG


@pytest.mark.parametrize("pos,off", [(0, 4), (1, 2), (2, 1), (4, 8), (5, 2)])
def test_combine_rejects_misaligned_pointers(pos, off):
    """Positions: 0 part_o, 1 part_m, 2 part_l, 4 out, 5 lse (3 is seq_lens)."""
    L = fd.lib()
    desc = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4)
    args = [_addr(i) for i in range(6)]
    args[pos] = _addr(pos, off)
    assert L.fd_decode_attn_combine(C.byref(desc), *args, None) == fd.FD_ERR_INVALID_ARG


@pytest.mark.parametrize("pos,off", [(0, 8), (1, 8), (2, 4), (5, 2), (7, 2), (8, 16), (10, 8), (11, 2),
                                     (13, 2)])
def test_paged_rejects_misaligned_pointers(pos, off):
    """Positions: 0 q, 1 k_cache, 2 v_cache, 5 block_table, 7 seq_lens,
    8 workspace (256 bytes), 10 out, 11 lse, 13 fallback_count."""
    L = fd.lib()
    desc = fd.make_desc(2, 8, 8, 128, "bf16", split_size=256, max_splits=4)
    ws = fd.fd_workspace_bytes(desc)
    args = [_addr(0), _addr(1), _addr(2), C.c_int32(64), C.c_int32(16), _addr(5), C.c_int32(64), _addr(7),
            _addr(8), C.c_size_t(ws), _addr(10), _addr(11), _addr(12), _addr(13)]
    args[pos] = _addr(pos, off)
    assert L.fd_decode_attn_paged(C.byref(desc), *args, None) == fd.FD_ERR_INVALID_ARG


def test_full_entry_point_validation():
    """fd_decode_attn: bad merge codes, misaligned pointers, a short workspace,
    and single-launch shapes beyond the counter area, all before any launch."""
    L = fd.lib()
    desc = fd.make_desc(2, 8, 8, 128, "bf16", split_size=256, max_splits=4)
    ws = fd.fd_workspace_bytes(desc)
    good = [_addr(0), _addr(1), _addr(2), C.c_int32(1024), _addr(4), _addr(5), C.c_size_t(ws), _addr(7), _addr(8),
            _addr(9), _addr(10)]

    def call(d, args):
        return L.fd_decode_attn(C.byref(d), *args, None)

    bad = fd.make_desc(2, 8, 8, 128, "bf16", split_size=256, max_splits=4)
    bad.merge = 3
    assert call(bad, good) == fd.FD_ERR_INVALID_ARG
    for pos, off in [(0, 8), (1, 4), (2, 2), (4, 2), (5, 16), (7, 8), (8, 2), (10, 2)]:
        args = list(good)
        args[pos] = _addr(pos, off)
        assert call(desc, args) == fd.FD_ERR_INVALID_ARG, pos
    args = list(good)
    args[6] = C.c_size_t(ws - 1)
    assert call(desc, args) == fd.FD_ERR_WORKSPACE_TOO_SMALL
    # 65535 requests x 2 KV heads: more (request, KV head) counters than the area holds
    big = fd.make_desc(65535, 2, 2, 128, "bf16", split_size=256, max_splits=1, merge="fused")
    args = list(good)
    args[6] = C.c_size_t(fd.fd_workspace_bytes(big))
    assert call(big, args) == fd.FD_ERR_UNSUPPORTED
    assert fd.fd_workspace_bytes(desc) == fd.TICKET_BYTES + 2 * 8 * 4 * 128 * 4 + 2 * 256


def test_whole_row_fallback_validation():
    """FD_FALLBACK_ROW needs flags (its second pass reads them) and the
    separate merge; an unknown fallback code is refused."""
    L = fd.lib()
    desc = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4, mode="unified", phi=-6.0, lo=-6.0, hi=6.0,
                        fallback="row")
    args = [_addr(i) for i in range(10)]
    args[3] = C.c_int32(16)
    args[8] = None                            # flags
    assert L.fd_decode_attn_partial(C.byref(desc), *args, None) == fd.FD_ERR_INVALID_ARG
    fused = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4, mode="unified", phi=-6.0, lo=-6.0, hi=6.0,
                         fallback="row", merge="fused")
    ws = fd.fd_workspace_bytes(fused)
    full = [_addr(0), _addr(1), _addr(2), C.c_int32(1024), _addr(4), _addr(5), C.c_size_t(ws), _addr(7), _addr(8),
            _addr(9), _addr(10)]
    assert L.fd_decode_attn(C.byref(fused), *full, None) == fd.FD_ERR_UNSUPPORTED
    bad = fd.make_desc(1, 8, 8, 128, "bf16", max_splits=4)
    bad.fallback = 2
    assert _partial_status(bad) == fd.FD_ERR_INVALID_ARG
