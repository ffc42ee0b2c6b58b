"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/dstopk.h declares, and rejects invalid calls before touching the device."""
import ctypes

import pytest

import top_selection_amd as ts

FAKE = 0x10000  # a 16-byte aligned address; never dereferenced by a rejected call


def test_exports_every_declared_symbol():
    names = ts.header_functions()
    assert {"ds_topk", "ds_topk_ex", "ds_topk_plan", "ds_topk_workspace_size", "ds_status_string",
            "ds_probe_read", "ds_probe_copy", "ds_probe_sink_words", "ds_topk_slices", "ds_topk_merge",
            "ds_topk_noalloc"} <= set(names)
    lib = ts.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, name in [(0, "DS_OK"), (-1, "DS_ERR_INVALID_ARG"), (-2, "DS_ERR_UNSUPPORTED"),
                       (-3, "DS_ERR_ALIGNMENT"), (-4, "DS_ERR_WORKSPACE"), (-5, "DS_ERR_LAUNCH"),
                       (-6, "DS_ERR_DEVICE")]:
        assert ts.ds_status_string(code) == name


def _call(x=FAKE, rows=4, n=1024, stride=None, k=8, dtype=ts.BF16, vals=FAKE, idx=FAKE, entry="ds_topk"):
    return getattr(ts.lib(), entry)(x, rows, n, n if stride is None else stride, k, dtype, 1, vals, idx, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), ts.DS_ERR_INVALID_ARG),
    (dict(k=1025, n=1024), ts.DS_ERR_INVALID_ARG),          # k > N
    (dict(k=4097, n=10000), ts.DS_ERR_UNSUPPORTED),          # k > 4096
    (dict(n=0), ts.DS_ERR_INVALID_ARG),
    (dict(n=2 ** 31), ts.DS_ERR_INVALID_ARG),
    (dict(rows=-1), ts.DS_ERR_INVALID_ARG),
    (dict(stride=1000), ts.DS_ERR_INVALID_ARG),             # row_stride < N
    (dict(dtype=2), ts.DS_ERR_INVALID_ARG),
    (dict(x=None), ts.DS_ERR_INVALID_ARG),
    (dict(vals=None, idx=None), ts.DS_ERR_INVALID_ARG),
    (dict(x=FAKE + 8), ts.DS_ERR_ALIGNMENT),
    (dict(n=1001, stride=1001), ts.DS_ERR_ALIGNMENT),        # 2002-byte rows
])
@pytest.mark.parametrize("entry", ["ds_topk", "ds_topk_noalloc"])
def test_rejects_before_launch(kw, code, entry):
    assert _call(entry=entry, **kw) == code


@pytest.mark.parametrize("entry", ["ds_topk", "ds_topk_noalloc"])
def test_empty_rows_is_a_no_op(entry):
    assert _call(rows=0, entry=entry) == ts.DS_OK


def test_noalloc_limit_matches_header():
    import re
    text = open(ts._binding.HEADER_PATH).read()
    m = re.search(r"#define DS_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ts.DS_NOALLOC_SCRATCH_BYTES


def test_workspace_rejected_without_touching_device():
    cfg = ts._binding.ds_config(0, 0, 4, 0)
    st = ts.lib().ds_topk_ex(FAKE, None, 2, 65536, 65536, 64, ts.BF16, 0, FAKE, FAKE, None, 0, ctypes.byref(cfg), None,
                             None)
    assert st == ts.DS_ERR_WORKSPACE


@pytest.mark.parametrize("dtype", [ts.BF16, ts.FP32])
@pytest.mark.parametrize("n,k,slices", [(32768, 512, 1), (131072, 512, 8), (129280, 512, 2), (1 << 20, 4096, 16),
                                        (268435456, 32, 512), (5000, 77, 3), (300, 300, 1)])
def test_forced_plans(dtype, n, k, slices):
    p = ts.ds_topk_plan(8, n, k, dtype, {"slices": slices})
    chunk = 512 if dtype == ts.BF16 else 256
    assert p["block"] % chunk == 0
    assert p["slices"] == slices
    assert p["slack"] >= 1
    per = -(-n // slices)
    assert p["slices"] == -(-n // (-(-per // p["block"]) * p["block"]))
    ws = ts.ds_topk_workspace_size(8, n, k, dtype, {"slices": slices})
    # split rows without the presampled start share a threshold word per row (8 rows: 64 bytes)
    shared = 64 if slices > 1 and p["presample"] == ts.PRESAMPLE_OFF else 0
    assert p["share"] == (ts.SHARE_AUTO if slices == 1 else (ts.SHARE_ON if shared else ts.SHARE_OFF))
    assert ws == shared + _list_merge_ws(8, slices, k)
    assert p["merge"] == (0 if slices == 1 else ts.MERGE_LISTS)
    sel = ts.ds_topk_workspace_size(8, n, k, dtype, {"slices": slices, "merge": ts.MERGE_SELECT})
    assert sel == (0 if slices == 1 else shared + 8 * ((slices * k + 1) // 2 * 2) * 8)


def _even(v):
    return (v + 1) // 2 * 2


def _merge_levels(slices, k):
    """Group sizes of the list merge's levels, from the rule the header states: at most 16
    lists and 128 KiB of 8-byte entries per group, the fewest levels, then per level the
    smallest group size that still reaches one list in the levels left."""
    gmax = min(16, (128 * 1024) // 8 // k)
    levels, reach = 0, 1
    while reach < slices:
        reach *= gmax
        levels += 1
    groups, lists = [], slices
    for lv in range(levels):
        g = 2
        while g ** (levels - lv) < lists:
            g += 1
        groups.append(g)
        lists = -(-lists // g)
    assert lists == 1 or slices == 1
    return groups


def _list_merge_ws(rows, slices, k):
    if slices == 1:
        return 0
    groups = _merge_levels(slices, k)
    ws = rows * _even(slices * k) * 8
    if len(groups) > 1:
        ws += rows * _even(-(-slices // groups[0]) * k) * 8
    return ws


def test_merge_levels_rule():
    assert _merge_levels(4, 512) == [4]
    assert _merge_levels(16, 512) == [16]
    assert _merge_levels(32, 512) == [6, 6]
    assert _merge_levels(33, 512) == [6, 6]
    assert _merge_levels(32, 4096) == [4, 3, 3]  # 32 -> 8 -> 3 -> 1
    assert _merge_levels(256, 32) == [16, 16]
    assert _merge_levels(512, 32) == [8, 8, 8]


def test_merge_plan_field():
    assert ts.ds_topk_plan(8, 1 << 20, 512, ts.BF16, {"slices": 32})["merge"] == ts.MERGE_LISTS
    assert ts.ds_topk_plan(8, 1 << 20, 512, ts.BF16, {"slices": 4})["merge"] == ts.MERGE_LISTS
    assert ts.ds_topk_plan(8, 1 << 20, 512, ts.BF16, {"slices": 32, "merge": ts.MERGE_SELECT})["merge"] == \
        ts.MERGE_SELECT
    assert ts.ds_topk_plan(8, 1 << 20, 512, ts.BF16, {"slices": 1, "merge": ts.MERGE_SELECT})["merge"] == 0
    with pytest.raises(ts.DSError) as e:
        ts.ds_topk_plan(4, 32768, 512, ts.BF16, {"merge": 3, "slices": 2})
    assert e.value.status == ts.DS_ERR_INVALID_ARG


def test_forced_block_sizes():
    assert ts.ds_topk_plan(4, 32768, 512, ts.BF16, {"block": 1024, "slack": 1024, "slices": 1})["waves"] == 2
    with pytest.raises(ts.DSError) as e:
        ts.ds_topk_plan(4, 32768, 512, ts.BF16, {"block": 1000, "slices": 1})
    assert e.value.status == ts.DS_ERR_UNSUPPORTED
    with pytest.raises(ts.DSError) as e:  # too many slices for the row: one would be empty
        ts.ds_topk_plan(1, 4096, 16, ts.FP32, {"slices": 64})
    assert e.value.status == ts.DS_ERR_UNSUPPORTED


def test_config_struct_matches_header():
    """The binding's ds_config has the header's fields in the header's order."""
    import re
    text = open(ts._binding.HEADER_PATH).read()
    body = re.search(r"typedef struct ds_config \{(.*?)\} ds_config;", text, re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [f for f, _ in ts._binding.ds_config._fields_]
    assert ctypes.sizeof(ts._binding.ds_config) == 4 * len(fields)


def test_presample_plan_field():
    on = ts.ds_topk_plan(64, 131072, 512, ts.BF16, {"slices": 4})
    assert on["presample"] == ts.PRESAMPLE_ON
    off = ts.ds_topk_plan(64, 131072, 512, ts.BF16, {"slices": 4, "presample": ts.PRESAMPLE_OFF})
    assert off["presample"] == ts.PRESAMPLE_OFF
    # k above 64 per wave of the workgroup: no presampled threshold
    big = ts.ds_topk_plan(8, 1 << 20, 4096, ts.BF16, {"slices": 8, "waves": 4})
    assert big["presample"] == ts.PRESAMPLE_OFF
    with pytest.raises(ts.DSError) as e:
        ts.ds_topk_plan(4, 32768, 512, ts.BF16, {"presample": 3, "slices": 1})
    assert e.value.status == ts.DS_ERR_INVALID_ARG


def test_order_group_plan_field():
    assert ts.ds_topk_plan(256, 129280, 512, ts.FP32, {"slices": 1})["order_group"] == 2  # 16 blocks
    assert ts.ds_topk_plan(64, 131072, 512, ts.BF16, {"slices": 4})["order_group"] == 1  # 4 blocks
    assert ts.ds_topk_plan(64, 131072, 512, ts.BF16, {"slices": 4, "order_group": 1})["order_group"] == 1
    with pytest.raises(ts.DSError) as e:
        ts.ds_topk_plan(4, 32768, 512, ts.BF16, {"order_group": 3, "slices": 1})
    assert e.value.status == ts.DS_ERR_INVALID_ARG


def test_schedule_plan_field():
    """The free-running schedule is the default unless B2 < B / 2; either can be forced;
    other values are rejected before any launch."""
    base = {"slices": 2}
    for n, k in ((100000, 64), (131072, 512), (1 << 20, 4096), (1 << 28, 32)):
        p = ts.ds_topk_plan(4, n, k, ts.BF16, base)
        want = ts.SCHEDULE_LOCKSTEP if 2 * p["slack"] < p["block"] else ts.SCHEDULE_FREE
        assert p["schedule"] == want, (n, k, p)
        assert ts.ds_topk_plan(4, n, k, ts.BF16, dict(base, schedule=ts.SCHEDULE_FREE))["schedule"] == \
            ts.SCHEDULE_FREE
    ix = ts.ds_topk_plan(4, 131072, 512, ts.BF16, {"slices": 4})  # the indexer: B2 near sqrt(k (k + B))
    assert (ix["block"], ix["slack"], ix["schedule"]) == (8192, 2048, ts.SCHEDULE_LOCKSTEP)
    assert ts.ds_topk_plan(4, 100000, 64, ts.BF16, dict(base, schedule=ts.SCHEDULE_LOCKSTEP))["schedule"] == \
        ts.SCHEDULE_LOCKSTEP
    with pytest.raises(ts.DSError) as e:
        ts.ds_topk_plan(4, 100000, 64, ts.BF16, dict(base, schedule=7))
    assert e.value.status == ts.DS_ERR_INVALID_ARG


def test_output_flags_in_plan():
    base = {"slices": 2}
    for flags in (0, ts.OUTPUT_UNSORTED, ts.OUTPUT_INDEX_INT64, ts.OUTPUT_UNSORTED | ts.OUTPUT_INDEX_INT64):
        assert ts.ds_topk_plan(4, 65536, 64, ts.BF16, dict(base, output=flags))["output"] == flags
    with pytest.raises(ts.DSError) as e:
        ts.ds_topk_plan(4, 65536, 64, ts.BF16, dict(base, output=4))
    assert e.value.status == ts.DS_ERR_INVALID_ARG


def test_warmup_in_plan():
    p = ts.ds_topk_plan(4, 65536, 64, ts.BF16, {"slices": 2, "warmup": 3})
    assert p["warmup"] == 3 and p["presample"] == ts.PRESAMPLE_OFF
    assert ts.ds_topk_plan(4, 65536, 64, ts.BF16, {"slices": 2})["warmup"] == 0
    with pytest.raises(ts.DSError) as e:
        ts.ds_topk_plan(4, 65536, 64, ts.BF16, {"slices": 2, "warmup": -1})
    assert e.value.status == ts.DS_ERR_INVALID_ARG


def test_share_in_plan():
    base = {"slices": 4}
    assert ts.ds_topk_plan(4, 65536, 64, ts.BF16, base)["share"] == ts.SHARE_OFF  # presampled start
    big = ts.ds_topk_plan(4, 1 << 20, 4096, ts.BF16, {"slices": 32})
    assert big["presample"] == ts.PRESAMPLE_OFF and big["share"] == ts.SHARE_ON
    assert ts.ds_topk_plan(4, 1 << 20, 4096, ts.BF16, {"slices": 32, "share": ts.SHARE_OFF})["share"] == ts.SHARE_OFF
    assert ts.ds_topk_plan(4, 65536, 64, ts.BF16, dict(base, share=ts.SHARE_ON))["share"] == ts.SHARE_ON
    assert ts.ds_topk_plan(4, 65536, 64, ts.BF16, {"slices": 1, "share": ts.SHARE_ON})["share"] == ts.SHARE_AUTO
    plain = ts.ds_topk_workspace_size(6, 65536, 64, ts.BF16, base)
    assert ts.ds_topk_workspace_size(6, 65536, 64, ts.BF16, dict(base, share=ts.SHARE_ON)) == plain + 48
    with pytest.raises(ts.DSError) as e:
        ts.ds_topk_plan(4, 65536, 64, ts.BF16, dict(base, share=3))
    assert e.value.status == ts.DS_ERR_INVALID_ARG
