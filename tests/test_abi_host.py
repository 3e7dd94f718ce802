"""The C-ABI library on the host: exported symbols, validation, planning and sizing (no GPU)."""
import ctypes
import re
import os

import numpy as np
import pytest

import speculative_decoding_draft_paged_amd as ba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "blockattn.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|void|const char\*)\s+(blockattn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = ba.load_library()
    names = header_functions()
    assert set(names) == set(ba.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layouts_match_header():
    # params: 14 int32 + 3 float = 68 bytes; info: 12 int32 + size_t = 56 bytes
    assert ctypes.sizeof(ba.blockattn_params) == 68
    assert ctypes.sizeof(ba.blockattn_plan_info_t) == 56


def params(**kw):
    base = dict(batch=2, block_size=7, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
                page_table_stride=4200, num_pages=9000, sm_scale=0.125)
    base.update(kw)
    return ba.make_params(**base)


def plan_info(prm, lens):
    plan = ba.blockattn_plan(prm, lens)
    info = plan.info()
    plan.destroy()
    return info


def test_host_only_plan_and_info():
    info = plan_info(params(), [131079, 131079])
    assert info["kind"] == 0 and info["uploaded"] == 0 and info["merge_active"] == 0
    assert info["units"] >= 256 and info["max_splits"] >= 64
    assert info["workspace_bytes"] == ba.blockattn_workspace_size(params(), [131079, 131079])


def test_split_heuristic_fills_the_gpu_and_bounds_partials():
    # one request, 128K keys, 2 kv heads: many splits; 32 requests x 16 heads: one split each
    small = plan_info(params(batch=1), [131079])
    assert small["units"] >= 240  # about one unit per CU (4097 tiles of each head in 125 splits)
    big = plan_info(params(batch=32, num_q_heads=64, num_kv_heads=16), [131079] * 32)
    assert big["max_splits"] == 1 and big["units"] == 512
    # every token group gets at least two tiles
    tiny = plan_info(params(batch=1), [200])
    assert tiny["max_splits"] == 1


def test_waves_override():
    assert plan_info(params(waves_override=8), [5000, 5000])["token_groups"] == 8
    assert plan_info(params(waves_override=1), [5000, 5000])["waves_per_unit"] == 1
    w = dict(head_dim=128, page_size=64, num_q_heads=16, num_kv_heads=1, window_left=4096, block_size=7)
    # R = 112 at D = 128 shares tiles: waves per workgroup = rows per wave choice, and a count
    # above the seven row blocks selects two token groups of four two-block waves
    info = plan_info(params(**w, waves_override=7), [8199, 8199])
    assert info["row_waves"] == 7 and info["token_groups"] == 1 and info["shared_tiles"] == 1
    info = plan_info(params(**w, waves_override=8), [8199, 8199])
    assert info["row_waves"] == 4 and info["token_groups"] == 2 and info["waves_per_unit"] == 8
    info = plan_info(params(**w, waves_override=4), [8199, 8199])
    assert info["row_waves"] == 4 and info["waves_per_unit"] == 4
    info = plan_info(params(**w, waves_override=1), [8199, 8199])
    assert info["row_waves"] == 4  # at most two row blocks per wave


def test_two_token_groups_for_many_row_blocks_and_tiles():
    """Seven or eight row blocks at D = 128 run as two token groups of four two-block waves
    once the batch holds at least 8 tiles per CU (2048 tiles); smaller batches keep one
    group of one-block waves."""
    w = dict(head_dim=128, page_size=64, num_q_heads=16, num_kv_heads=1, window_left=4096, window_right=-1)
    for K, blocks in ((7, 7), (8, 8)):
        n = 16384 + K  # 129 tiles of the window per request
        small = plan_info(params(**w, block_size=K, batch=15), [n] * 15)  # 1935 tiles
        big = plan_info(params(**w, block_size=K, batch=16), [n] * 16)    # 2064 tiles
        assert small["token_groups"] == 1 and small["row_waves"] == blocks
        assert big["token_groups"] == 2 and big["row_waves"] == 4 and big["waves_per_unit"] == 8
    # five and six blocks keep one group at any size
    info = plan_info(params(**w, block_size=5, batch=64), [16389] * 64)
    assert info["token_groups"] == 1 and info["row_waves"] == 5


def test_three_blocks_two_token_groups_with_fp8_pools_and_many_tiles():
    """Three row blocks at D = 128 (R = 48): four one-block waves, one rowless. With fp8 pools
    and at least 64 tiles per CU (16384 tiles) they run as two token groups; bf16 pools and
    smaller batches keep one group; a wave count above the blocks forces two groups."""
    w = dict(head_dim=128, page_size=64, num_q_heads=64, num_kv_heads=4, block_size=3, window_left=4096,
             window_right=-1, page_table_stride=300, num_pages=64 * 300)
    n = 16384 + 3  # 129 window tiles per (request, kv head)
    fp8_big = plan_info(params(**w, batch=32, kv_dtype="fp8_e4m3"), [n] * 32)    # 16512 tiles
    fp8_small = plan_info(params(**w, batch=31, kv_dtype="fp8_e4m3"), [n] * 31)  # 15996 tiles
    bf16_big = plan_info(params(**w, batch=32), [n] * 32)
    forced = plan_info(params(**w, batch=2, waves_override=8), [n] * 2)
    assert fp8_big["token_groups"] == 2 and fp8_big["row_waves"] == 4 and fp8_big["waves_per_unit"] == 8
    for info in (fp8_small, bf16_big):
        assert info["token_groups"] == 1 and info["row_waves"] == 4 and info["waves_per_unit"] == 4
    assert forced["token_groups"] == 2 and forced["row_waves"] == 4


def test_co_resident_workgroups_share_a_cu_in_the_split_choice():
    """Four one-block waves at R = 48 fit two workgroups on a CU, but those share the CU's
    throughput: 64 requests of 129 tiles take one unit per CU (4 splits, 256 units), not
    two (8 splits, 512 units), and the mixed-length windowed batch keeps its requests whole."""
    w = dict(head_dim=128, page_size=64, num_q_heads=16, num_kv_heads=1, block_size=3, window_left=4096,
             window_right=-1, page_table_stride=300, num_pages=64 * 300)
    info = plan_info(params(**w, batch=64), [16384 + 3] * 64)
    assert info["units"] == 256 and info["max_splits"] == 4
    lens = [2048 + 3 + (i * 977) % 14337 for i in range(64)]
    info = plan_info(params(**dict(w, num_q_heads=64, num_kv_heads=4), batch=64), lens)
    assert info["units"] == 256 and info["max_splits"] == 1


def test_streaming_units_hold_16k_of_keys_and_values_per_wave():
    """The split choice's floor: two 32-token tiles per wave at D = 64 (eight waves: 16
    tiles per unit), one at D = 128 (four waves: 4 tiles per unit)."""
    d128 = dict(head_dim=128, page_size=64, num_q_heads=16, num_kv_heads=1, block_size=1, window_left=4096,
                window_right=-1, page_table_stride=300, num_pages=300)
    info = plan_info(params(**d128, batch=1), [16384 + 1])  # 129 window tiles
    assert info["shared_tiles"] == 0 and info["max_splits"] == 33
    info = plan_info(params(page_table_stride=1100, batch=1), [32768 + 7])  # 1025 tiles at D = 64
    assert info["shared_tiles"] == 0 and info["max_splits"] == 65


def test_tile_kernel_choice():
    # R <= 32: one row-wave, waves stream their own tiles; more rows share tiles through LDS
    assert plan_info(params(), [5000, 5000])["shared_tiles"] == 0
    info = plan_info(params(num_q_heads=16, num_kv_heads=1, block_size=3), [5000, 5000])  # R = 48, D = 64
    assert info["shared_tiles"] == 1 and info["row_waves"] == 2 and info["waves_per_unit"] == 2
    w = dict(head_dim=128, page_size=64, num_q_heads=16, num_kv_heads=1, window_left=4096)
    info = plan_info(params(**w, block_size=5), [8197, 8197])  # R = 80: one row block per wave
    assert info["shared_tiles"] == 1 and info["row_waves"] == 5 and info["token_groups"] == 1
    info = plan_info(params(**w, block_size=3), [8195, 8195])  # R = 48: one block per wave, plus a rowless wave
    assert info["shared_tiles"] == 1 and info["row_waves"] == 4 and info["waves_per_unit"] == 4
    info = plan_info(params(**w, block_size=3, waves_override=3), [8195, 8195])  # three waves, no rowless one
    assert info["shared_tiles"] == 1 and info["row_waves"] == 3
    info = plan_info(params(**w, block_size=3, waves_override=2), [8195, 8195])  # two blocks per wave
    assert info["shared_tiles"] == 1 and info["row_waves"] == 2
    assert plan_info(params(**w, block_size=1), [8193, 8193])["shared_tiles"] == 0  # R = 16


def test_more_than_128_rows_run_as_row_groups():
    w = dict(head_dim=128, page_size=64)
    one = plan_info(params(**w, block_size=8, num_q_heads=16, num_kv_heads=1), [4000, 4000])  # R = 128
    two = plan_info(params(**w, block_size=16, num_q_heads=16, num_kv_heads=1), [4000, 4000])  # R = 256
    three = plan_info(params(**w, block_size=9, num_q_heads=32, num_kv_heads=2), [4000, 4000])  # R = 144
    assert one["row_groups"] == 1 and two["row_groups"] == 2 and three["row_groups"] == 2
    # 128-row groups of eight one-block waves (a small batch); 144 rows: two row groups of
    # five row blocks
    assert two["row_waves"] == 8 and two["token_groups"] == 1
    assert three["row_waves"] == 5 and three["token_groups"] == 1
    # every row group gets the same split count, so the units scale with the groups
    forced = [plan_info(params(**w, block_size=k, num_q_heads=16, num_kv_heads=1, splits_override=3), [4000, 4000])
              for k in (8, 16)]
    assert forced[0]["units"] == 2 * 3 and forced[1]["units"] == 2 * 3 * 2
    big = plan_info(params(**w, block_size=16, num_q_heads=64, num_kv_heads=2, batch=1), [9000])  # R = 512
    assert big["row_groups"] == 4 and big["shared_tiles"] == 1


def test_splits_override_and_clamp():
    info = plan_info(params(batch=1, splits_override=5), [1000])
    assert info["max_splits"] == 5 and info["units"] == 10
    info = plan_info(params(batch=1, splits_override=10 ** 6), [1000])
    assert info["max_splits"] == (1000 + 31) // 32


def test_windowed_plan_merge_flag():
    w = dict(head_dim=128, page_size=64, num_q_heads=16, num_kv_heads=1, window_left=4096)
    assert plan_info(params(**w, block_size=7, window_right=-1), [8199, 8199])["merge_active"] == 1
    assert plan_info(params(**w, block_size=1, window_right=-1), [8193, 8193])["merge_active"] == 0
    assert plan_info(params(**w, block_size=7, window_right=0), [8199, 8199])["merge_active"] == 0
    info = plan_info(params(**w, block_size=7, window_right=-1), [8199, 8199])
    assert info["kind"] == 1 and info["row_waves"] == 7


@pytest.mark.parametrize("B", [1, 2, 32, 33, 200])
def test_workspace_size_grows_with_batch(B):
    lens = np.full(B, 32775, np.int32)
    nbytes = ba.blockattn_workspace_size(params(batch=B, page_table_stride=1100), lens)
    info = plan_info(params(batch=B, page_table_stride=1100), lens)
    R, D = 28, 64
    floats = info["units"] * R * (D + 2) * 4
    assert floats <= nbytes <= floats + info["units"] * 16 + B * 2 * (8 + 4) + 6 * 256


@pytest.mark.parametrize("kw,lens,code,needle", [
    (dict(head_dim=96), [100, 100], ba.BLOCKATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(num_pages=2 ** 30), [100, 100], ba.BLOCKATTN_ERR_UNSUPPORTED, "num_pages * num_kv_heads"),
    (dict(kv_dtype=7), [100, 100], ba.BLOCKATTN_ERR_UNSUPPORTED, "kv_dtype"),
    (dict(kv_dtype="fp8_e4m3", k_scale=0.0), [100, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "k_scale"),
    (dict(k_scale=float("inf")), [100, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "k_scale"),
    (dict(v_scale=float("nan")), [100, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "v_scale"),
    (dict(page_size=48), [100, 100], ba.BLOCKATTN_ERR_UNSUPPORTED, "page_size"),
    (dict(page_size=8), [100, 100], ba.BLOCKATTN_ERR_UNSUPPORTED, "page_size"),
    (dict(page_size=512), [100, 100], ba.BLOCKATTN_ERR_UNSUPPORTED, "page_size"),
    (dict(num_q_heads=7), [100, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "num_q_heads"),
    (dict(block_size=17), [100, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "block_size"),
    (dict(), [6, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "seq_lens[0]"),
    (dict(page_table_stride=3), [100, 97], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "page_table_stride"),
    (dict(window_left=0), [100, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "window_left"),
    (dict(window_right=3), [100, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "window_right"),
    (dict(sm_scale=float("nan")), [100, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "sm_scale"),
    (dict(waves_override=9), [100, 100], ba.BLOCKATTN_ERR_INVALID_ARGUMENT, "waves_override"),
])
def test_invalid_parameters_are_named(kw, lens, code, needle):
    with pytest.raises(ba.BlockAttnError) as e:
        ba.blockattn_plan(params(**kw), lens)
    assert e.value.status == code
    assert needle in e.value.message


def test_forward_refuses_plans_without_workspace_or_wrong_kind():
    lib = ba.load_library()
    plan = ba.blockattn_plan(params(), [100, 100])
    vp = ctypes.c_void_p
    one = vp(0x1000)
    rc = lib.blockattn_forward(vp(plan.handle), one, one, one, one, one, one, one, None, None)
    assert rc == ba.BLOCKATTN_ERR_PLAN_MISMATCH and "workspace" in ba.blockattn_last_error()
    rc = lib.blockattn_windowed_forward(vp(plan.handle), one, one, one, one, one, one, one, one, None)
    assert rc == ba.BLOCKATTN_ERR_PLAN_MISMATCH and "blockattn_forward" in ba.blockattn_last_error()
    plan.destroy()


def test_scratch_forward_refuses_plans_larger_than_the_array():
    """A plan whose work list and partials exceed the scratch array is refused before any HIP call."""
    lib = ba.load_library()
    # 16 requests x 2 kv heads x 1000 forced splits of 28 rows: about 115 MB of partials
    prm = ba.make_params(batch=16, block_size=7, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
                         page_table_stride=2000, num_pages=40000, sm_scale=0.125, splits_override=1000)
    lens = np.full(16, 40000, np.int32)
    assert ba.blockattn_workspace_size(prm, lens) > ba.BLOCKATTN_SCRATCH_BYTES
    plan = ba.blockattn_plan(prm, lens)
    vp = ctypes.c_void_p
    one = vp(0x1000)
    rc = lib.blockattn_forward_scratch(vp(plan.handle), one, one, one, one, one, one, None, None)
    assert rc == ba.BLOCKATTN_ERR_WORKSPACE_TOO_SMALL and "scratch" in ba.blockattn_last_error()
    rc = lib.blockattn_forward_scratch(None, one, one, one, one, one, one, None, None)
    assert rc == ba.BLOCKATTN_ERR_INVALID_ARGUMENT
    plan.destroy()
    # a windowed plan that fits still needs its lse
    ok = ba.blockattn_plan(params(window_left=64), [100, 100])
    rc = lib.blockattn_forward_scratch(vp(ok.handle), one, one, one, one, one, one, None, None)
    assert rc == ba.BLOCKATTN_ERR_INVALID_ARGUMENT and "lse" in ba.blockattn_last_error()
    ok.destroy()


def test_forward_block_checks_its_own_arguments_first():
    lib = ba.load_library()
    vp = ctypes.c_void_p
    one = vp(0x1000)

    def call(plan, kb, vb, append=0):
        return lib.blockattn_forward_block(vp(plan.handle), one, kb, vb, one, one, one, one, None, one, one,
                                           ctypes.c_int32(append), None)

    plan = ba.blockattn_plan(params(), [100, 100])
    assert call(plan, None, one) == ba.BLOCKATTN_ERR_INVALID_ARGUMENT
    assert "k_block" in ba.blockattn_last_error()
    assert call(plan, one, one) == ba.BLOCKATTN_ERR_PLAN_MISMATCH and "workspace" in ba.blockattn_last_error()
    plan.destroy()
    for vs in (0.0, 1e-39, -1e-39):  # no finite fp32 reciprocal
        plan = ba.blockattn_plan(params(kv_dtype="fp8_e4m3", v_scale=vs), [100, 100])
        assert call(plan, one, one) == ba.BLOCKATTN_ERR_INVALID_ARGUMENT
        assert "v_scale" in ba.blockattn_last_error()
        plan.destroy()


def test_fp8_plan_keeps_the_bf16_shape():
    """The element type changes only the loads: same kernel shape, units and workspace."""
    for kw in (dict(), dict(head_dim=128, page_size=64, num_q_heads=16, num_kv_heads=1, window_left=4096,
                            block_size=7)):
        a = plan_info(params(**kw), [9000, 5000])
        b = plan_info(params(**kw, kv_dtype="fp8_e4m3", k_scale=0.0625, v_scale=0.0625), [9000, 5000])
        assert a == b


def test_merge_checks_its_arguments():
    lib = ba.load_library()
    vp = ctypes.c_void_p
    one, two = vp(0x1000), vp(0x100000)

    def call(parts, rows, d, po=one, pl=one, out=two):
        return lib.blockattn_merge(ctypes.c_int32(parts), ctypes.c_int64(rows), ctypes.c_int32(d), po, pl, out, None,
                                   None)

    assert call(0, 10, 64) == ba.BLOCKATTN_ERR_INVALID_ARGUMENT and "parts" in ba.blockattn_last_error()
    assert call(2, -1, 64) == ba.BLOCKATTN_ERR_INVALID_ARGUMENT
    assert call(2, 10, 96) == ba.BLOCKATTN_ERR_UNSUPPORTED and "head_dim" in ba.blockattn_last_error()
    assert call(2, 0, 64, None, None, None) == ba.BLOCKATTN_OK  # nothing to merge, nothing launched
    assert call(2, 10, 64, one, one, None) == ba.BLOCKATTN_ERR_INVALID_ARGUMENT
    assert call(2, 10, 64, one, one, vp(0x1000 + 64)) == ba.BLOCKATTN_ERR_INVALID_ARGUMENT  # overlaps part_out
    assert "overlap" in ba.blockattn_last_error()


def test_combine_mode_plan_choice():
    lens = [131079, 131079]
    auto = plan_info(params(page_table_stride=4200), lens)
    assert auto["max_splits"] > 1 and auto["fused_combine"] == 0 and auto["combine_launch"] == 1
    last = plan_info(params(page_table_stride=4200, combine="last_arriver"), lens)
    assert last["fused_combine"] == 1 and last["combine_launch"] == 0
    kern = plan_info(params(page_table_stride=4200, combine="kernel"), lens)
    assert kern["fused_combine"] == 0 and kern["combine_launch"] == 1
    # one split per request: nothing to combine, whatever the mode
    one = plan_info(params(page_table_stride=4200, combine="last_arriver", splits_override=1), lens)
    assert one["fused_combine"] == 0 and one["combine_launch"] == 0
    # the in-kernel combine folds each item's splits in registers (only its arrival flag sits in
    # LDS), so any split count is accepted
    many = plan_info(params(page_table_stride=4200, combine="last_arriver", splits_override=4000), lens)
    assert many["fused_combine"] == 1 and many["max_splits"] == 4000
    with pytest.raises(ba.BlockAttnError) as e:
        ba.blockattn_plan(params(combine=3), [100, 100])
    assert e.value.status == ba.BLOCKATTN_ERR_INVALID_ARGUMENT and "combine_mode" in e.value.message
