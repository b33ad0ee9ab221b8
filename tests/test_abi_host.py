"""Host-side checks of libmoe_shard.so (no GPU needed, no kernel launches).

The library must load, export every function the headers under include/ declare,
and reject invalid problems on the host with the documented status codes
before touching the GPU.  Buffer bounds follow the pages' capacity rules.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _binding():
    lib = os.path.join(ROOT, "grouped_gemm_shard_amd", "libmoe_shard.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "gg_build", os.path.join(ROOT, "grouped_gemm_shard_amd", "build.py"))
        m = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(m)
        m.build()
    import grouped_gemm_shard_amd as g
    return g


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            text = open(os.path.join(inc, h)).read()
            names |= set(re.findall(r"^(?:int|const char\*)\s+(moe_\w+)\(", text, re.M))
    return sorted(names)


def test_exports_match_header():
    g = _binding()
    decl = declared_functions()
    assert sorted(g.EXPORTED) == decl
    lib = ctypes.CDLL(g.lib_path)
    for name in decl:
        assert hasattr(lib, name), name


def problem(**kw):
    g = _binding()
    base = dict(tokens=4096, seq_len=4096, hidden=1024, ffn=512, num_experts=32, top_k=4,
                num_shards=8, res_lo=0, res_hi=8, factor=1.5, num_chunks=4)
    base.update(kw)
    return g.Problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(tokens=0), -1), (dict(seq_len=1000), -1), (dict(num_experts=30), -1),
    (dict(top_k=0), -1), (dict(top_k=33, num_experts=64), -2), (dict(res_lo=3, res_hi=3), -1),
    (dict(res_hi=9), -1), (dict(num_chunks=3), -1), (dict(hidden=1000), -2),
    (dict(ffn=100), -2), (dict(slots_per_shard=1, num_replicas=9), -1),
    (dict(slots_per_shard=1, num_replicas=2, res_hi=4), -2),
    (dict(num_experts=2048, num_shards=8), -2), (dict(factor=float("nan")), -1),
    (dict(num_chunks=0, factor=1.5), -1),   # ceil(8 / 1.5) = 6 does not divide 4096
])
def test_invalid_problems_rejected(kw, status):
    g = _binding()
    with pytest.raises(g.MoeError) as ei:
        g.layer_workspace_bytes(problem(**kw), g.MODE_LAYER)
    assert ei.value.status == status


def test_invalid_gate_and_mode():
    g = _binding()
    c = problem().c()
    c.gate = 7
    size = ctypes.c_size_t()
    assert g.lib.moe_layer_workspace_bytes(ctypes.byref(c), 0, ctypes.byref(size)) == -1
    assert g.lib.moe_layer_workspace_bytes(ctypes.byref(problem().c()), 9,
                                           ctypes.byref(size)) == -1


def test_null_pointers_rejected_before_launch():
    g = _binding()
    c = problem().c()
    assert g.lib.moe_route(ctypes.byref(c), None, None, None, None) == -1
    assert g.lib.moe_layer_dropless_chunked(ctypes.byref(c), 0, None, None, None, None, None,
                                            None, None, None, 0, None) == -1
    assert g.lib.moe_status_string(-3).decode() == "buffer or workspace too small"


def test_return_path_dedup_entry_points_validate_on_the_host():
    g = _binding()
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    plain = problem().c()
    dd_p = problem(dedup=True)
    dd = dd_p.c()
    rows, drows = g.pass_max_rows(dd_p, 1, 0)
    part = lambda c, n, ch, cap, eo, mr, md: g.lib.moe_combine_partial(  # noqa: E731
        ctypes.byref(c), n, ch, cap, eo, fake, fake, fake, fake, fake, fake, mr, md, None)
    src = lambda c, n, ch, cap, pa, mr, md: g.lib.moe_combine_from_partials(  # noqa: E731
        ctypes.byref(c), n, ch, cap, pa, fake, fake, fake, mr, md, None)
    # without dedup there are no partial rows
    assert part(plain, 1, 0, 0, fake, rows, drows) == -1
    assert src(plain, 1, 0, 0, fake, rows, drows) == -1
    # null arrays, negative bounds, a chunk outside the chunk count, bad capped
    assert part(dd, 1, 0, 0, None, rows, drows) == -1
    assert part(dd, 1, 0, 0, fake, -1, drows) == -1
    assert src(dd, 4, 4, 0, fake, rows, drows) == -1
    assert src(dd, 1, 0, 2, fake, rows, drows) == -1
    # misaligned rows
    assert part(dd, 1, 0, 0, ctypes.c_void_p(258), rows, drows) == -1
    # buffers below the pass's worst case: never a silent truncation
    assert part(dd, 1, 0, 0, fake, rows, drows - 1) == -3
    assert src(dd, 1, 0, 0, fake, rows - 1, drows) == -3

def test_pass_row_bounds():
    g = _binding()
    # Llama4-Maverick shard: cap = 2 * 32768 / 16 = 4096; a chunk of 4096
    # tokens has a worst case of 4096 rows per shard, no more than the cap
    # (the fallback page, How: a chunk's worst-case buffer fits within the
    # capped one).
    mav = problem(tokens=32768, seq_len=8192, hidden=5120, ffn=8192, num_experts=128, top_k=1,
                  num_shards=16, res_lo=0, res_hi=1, factor=2.0, num_chunks=8, gate="sigmoid")
    assert g.pass_max_rows(mav, 8, 0) == (4096, 0)
    assert g.pass_max_rows(mav, 1, 1) == (4096, 0)
    assert g.pass_max_rows(mav, 1, 0) == (32768, 0)
    # mid layer: capped 8 shards x 3072; a chunk of 1024 tokens x 4 rows
    mid = problem()
    assert g.pass_max_rows(mid, 1, 1) == (16384, 0)
    assert g.pass_max_rows(mid, 4, 0) == (4096, 0)
    # dedup: unique rows per shard bounded by the chunk's tokens and the cap
    ded = problem(tokens=8192, seq_len=8192, hidden=7168, ffn=2048, num_experts=256, top_k=8,
                  num_shards=16, res_lo=0, res_hi=16, factor=2.0, num_chunks=8, dedup=True,
                  slots_per_shard=2, num_replicas=2)
    assert g.pass_max_rows(ded, 1, 0) == (65536, 65536)
    assert g.pass_max_rows(ded, 8, 0) == (8192, 8192)


def test_layer_workspace_grows_with_uncapped_modes():
    g = _binding()
    p = problem()
    capped = g.layer_workspace_bytes(p, g.MODE_CAPPED_ONLY)
    dropless = g.layer_workspace_bytes(p, g.MODE_FORCE_DROPLESS)
    chunked = g.layer_workspace_bytes(p, g.MODE_FORCE_CHUNKED)
    layer = g.layer_workspace_bytes(p, g.MODE_LAYER)
    assert chunked < capped <= dropless
    assert layer == max(capped, chunked) or layer >= capped
    assert g.workspace_bytes(p) > 0


def test_fallback_chunks_per_pass_stay_within_the_capped_buffer():
    g = _binding()
    # One resident shard (Llama4-Maverick shard): a chunk's worst case already
    # equals the capped buffer, which would leave 8 passes of one chunk, so
    # the pass buffers hold twice that and the passes two chunks each.
    mav = problem(tokens=32768, seq_len=8192, hidden=5120, ffn=8192, num_experts=128, top_k=1,
                  num_shards=16, res_lo=0, res_hi=1, factor=2.0, num_chunks=8, gate="sigmoid")
    assert g.layer_chunks_per_pass(mav, g.MODE_LAYER) == 2
    # All 8 virtual shards resident (mid layer): the buffer of 8 x 3072 rows
    # holds every assignment (16384 rows), so the 4 chunks run together.
    mid = problem()
    assert g.layer_chunks_per_pass(mid, g.MODE_LAYER) == 4
    # FORCE_CHUNKED is sized for one chunk, doubled for its 4 passes.
    assert g.layer_chunks_per_pass(mid, g.MODE_FORCE_CHUNKED) == 2
    # dedup + redundancy over 16 resident shards: rows and dedup rows of all
    # 8 chunks (65536 each) fit the capped bounds.
    ded = problem(tokens=8192, seq_len=8192, hidden=7168, ffn=2048, num_experts=256, top_k=8,
                  num_shards=16, res_lo=0, res_hi=16, factor=2.0, num_chunks=8, dedup=True,
                  slots_per_shard=2, num_replicas=2)
    assert g.layer_chunks_per_pass(ded, g.MODE_LAYER) == 8
    # DeepSeek-V3 shard, 1 of 8 resident: cap 8192 = one chunk's worst case,
    # doubled for the fallback's passes.
    ds = problem(tokens=4096, seq_len=4096, hidden=7168, ffn=2048, num_experts=256, top_k=8,
                 num_shards=8, res_lo=0, res_hi=1, factor=2.0, num_chunks=4)
    assert g.layer_chunks_per_pass(ds, g.MODE_LAYER) == 2
    # the chunks of a pass divide num_chunks here
    for p, n in ((mav, 8), (mid, 4), (ded, 8), (ds, 4)):
        q = g.layer_chunks_per_pass(p, g.MODE_LAYER)
        assert n % q == 0
        rows_q, drows_q = g.pass_max_rows(p, n // q, 0)
        r1, u1 = g.pass_max_rows(p, 1, 1)
        rc, uc = g.pass_max_rows(p, n, 0)
        # one pass: within the capped buffer; passes of a multi-pass call:
        # within twice it
        k = 1 if q == n else 2
        assert rows_q <= k * max(r1, rc) and drows_q <= k * max(u1, uc)


def test_two_chunk_passes_hold_twice_the_capped_rows():
    # the Maverick shard's passes of two chunks: twice the rows of the capped
    # buffer (a chunk's worst case equals it)
    g = _binding()
    mav = problem(tokens=32768, seq_len=8192, hidden=5120, ffn=8192, num_experts=128, top_k=1,
                  num_shards=16, res_lo=0, res_hi=1, factor=2.0, num_chunks=8, gate="sigmoid")
    rows1, _ = g.pass_max_rows(mav, 1, 1)
    rows8, _ = g.pass_max_rows(mav, 8, 0)
    rows4, _ = g.pass_max_rows(mav, 4, 0)
    assert rows4 == 2 * max(rows1, rows8)


def test_backward_entry_points_validate_on_the_host():
    g = _binding()
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    c = problem().c()
    rows = 16384
    need = g.bwd_workspace_bytes(problem(), rows)
    # scratch: tile offsets, d_a, d_hg|d_hu and the recomputed activation,
    # 4F bf16 values per row
    assert need >= rows * 4 * 512 * 2
    gmm = lambda cc, acc, mr, ws, nb, wd=fake: g.lib.moe_gmm_swiglu_bwd(  # noqa: E731
        ctypes.byref(cc), fake, fake, fake, fake, fake, wd, fake, fake, fake, fake, fake, acc, mr,
        ws, nb, None)
    assert gmm(c, 0, rows, None, need) == -1          # no workspace
    assert gmm(c, 2, rows, fake, need) == -1          # accumulate is 0 or 1
    assert gmm(c, 0, -1, fake, need) == -1            # negative rows
    assert gmm(c, 0, rows, fake, need, None) == -1    # no down weights
    assert gmm(c, 0, rows, ctypes.c_void_p(128), need) == -1  # ws alignment
    assert gmm(c, 0, rows, fake, need - 1) == -3      # workspace too small
    # 32-bit buffer offsets: rows * max(H, 2F) * 2 bytes must stay below 2^31
    assert gmm(c, 0, 1 << 20, fake, 1 << 40) == -2
    assert g.lib.moe_combine_bwd(ctypes.byref(c), 4, 4, fake, fake, fake, fake, fake, fake, rows,
                                 None) == -1
    assert g.lib.moe_combine_bwd(ctypes.byref(c), 1, 0, ctypes.c_void_p(258), fake, fake, fake,
                                 fake, fake, rows, None) == -1
    assert g.lib.moe_permute_bwd(ctypes.byref(c), 1, 0, None, fake, fake, rows, None) == -1
    assert g.lib.moe_route_bwd(ctypes.byref(c), fake, None, fake, fake, None) == -1


def test_layer_backward_validates_on_the_host():
    g = _binding()
    fake = ctypes.c_void_p(256)
    c = problem().c()
    need = g.layer_bwd_workspace_bytes(problem(), g.MODE_LAYER)
    assert need > g.layer_workspace_bytes(problem(), g.MODE_LAYER)
    call = lambda mode, ws, nb, dy=fake: g.lib.moe_layer_bwd(  # noqa: E731
        ctypes.byref(c), mode, fake, fake, fake, fake, fake, dy, fake, fake, fake, fake, fake, ws,
        nb, None)
    assert call(9, fake, need) == -1        # mode
    assert call(0, fake, need, None) == -1  # no upstream gradient
    assert call(0, None, need) == -1        # no workspace
    assert call(0, fake, need - 1) == -3    # workspace too small


def test_calib_rejects_bad_arguments_on_the_host():
    """The calibration entry points validate before any launch."""
    g = _binding()
    L = g._lib()
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert L.moe_calib_copy(p, None, 16, 1, None) == -1           # null destination
    assert L.moe_calib_copy(p, p, 24, 1, None) == -1               # not a multiple of 16
    assert L.moe_calib_copy(p, p, 16, 0, None) == -1               # no workgroups
    f = ctypes.c_int64()
    assert L.moe_calib_mfma(0, 1, p, ctypes.byref(f), None) == -1  # no workgroups
    assert L.moe_calib_mfma(1, 1, None, ctypes.byref(f), None) == -1
