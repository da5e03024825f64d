"""The C-ABI library loads and exports every symbol its headers declare;
host-side argument validation (no GPU needed: nothing is launched)."""
import ctypes
import os
import re

import pytest

from hash_table_amd import tsdf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("tsdf.h", "tsdf_microbench.h")]


def declared_functions():
    names = []
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(tsdf_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_headers_match_binding():
    assert declared_functions() == sorted(tsdf.EXPORTS)


@pytest.mark.parametrize("name", declared_functions())
def test_symbol_exported(name):
    lib = ctypes.CDLL(tsdf.LIBRARY)
    assert hasattr(lib, name)


def test_table_sizing_rule():
    # smallest power of two at or above twice the pool: at most half full
    assert tsdf.tsdf_table_entries_for(4096) == 8192
    assert tsdf.tsdf_table_entries_for(65536) == 131072
    assert tsdf.tsdf_table_entries_for(3) == 8
    assert tsdf.tsdf_table_entries_for(1 << 22) == 1 << 23
    assert tsdf.tsdf_table_entries_for(0) == -1
    assert tsdf.tsdf_table_entries_for(tsdf.TSDF_MAX_POOL_BLOCKS + 1) == -1
    assert tsdf.tsdf_counters_bytes() == 64 * 640 + 96 * 104     # statistics + 96 frames of launch parameters


def test_scratch_sizing():
    def expect(entries, px):
        part_px = max(-(-px // 64), 256)                            # a partition holds at least a 16 x 16 tile
        seg_part, rec_part = 2 * part_px, 4 * part_px                 # 2 segments, 4 runs per pixel
        item_part = max(64, entries // 32)
        counters = 64 * 128 + 128 + 8 * 32 * 4                      # per frame parity: partitions, totals, XCD fetch
        units = 8 * 8192                                              # split-block work units
        return (2 * counters + 32 * entries + 16 * 64 * seg_part + 12 * 64 * rec_part + units + 8 * 64 * seg_part
                + 8 * entries + 4 * 64 * item_part + 12 * entries)
    owner = tsdf.tsdf_config(0.01, 0.04, 4096, 0, tsdf.TSDF_UPDATE_OWNER, 1000)
    assert tsdf.tsdf_scratch_bytes(owner) == expect(8192, 1000)
    default = tsdf.tsdf_config(0.01, 0.04, 4096, 0, tsdf.TSDF_UPDATE_OWNER, 0)
    assert tsdf.tsdf_scratch_bytes(default) == expect(8192, 1 << 20)
    rays = tsdf.tsdf_config(0.01, 0.04, 4096, 0, tsdf.TSDF_UPDATE_RAYS)
    assert tsdf.tsdf_scratch_bytes(rays) == 0
    bad = tsdf.tsdf_config(0.01, 0.04, 0, 0, tsdf.TSDF_UPDATE_OWNER)
    assert tsdf.tsdf_scratch_bytes(bad) == 0


def test_status_strings():
    assert [tsdf.tsdf_status_str(s) for s in (0, -1, -2, -3, -4, -5, 7)] == [
        "TSDF_OK", "TSDF_EINVAL", "TSDF_EALIGN", "TSDF_EHIP", "TSDF_ESMALL", "TSDF_ELIMIT", "TSDF_UNKNOWN"]


def _buffers(base=0x10000, step=0x100000):
    return tsdf.tsdf_buffers(*(base + i * step for i in range(8)))


@pytest.mark.parametrize("cfg,code", [
    ((0.0, 0.04, 4096, 0), tsdf.TSDF_EINVAL),               # voxel size
    ((0.01, float("nan"), 4096, 0), tsdf.TSDF_EINVAL),      # truncation
    ((0.01, 0.04, 0, 0), tsdf.TSDF_EINVAL),                 # empty pool
    ((0.01, 0.04, 4096, 6000), tsdf.TSDF_EINVAL),           # table not a power of two
    ((0.01, 0.04, 4096, 4096), tsdf.TSDF_EINVAL),           # table under twice the pool
    ((0.01, 0.04, 1 << 31, 0), tsdf.TSDF_EINVAL),           # pool too large
    ((0.01, 0.04, 4096, 0, 7), tsdf.TSDF_EINVAL),           # unknown update mode
    ((0.01, 0.04, 4096, 0, 0, -5), tsdf.TSDF_EINVAL),       # negative frame size
    ((0.01, 0.04, 4096, 0, 0, 0, -1), tsdf.TSDF_EINVAL),    # negative probe limit
])
def test_create_rejects_bad_config(cfg, code):
    with pytest.raises(tsdf.TsdfError) as e:
        tsdf.tsdf_create(tsdf.tsdf_config(*cfg), _buffers())
    assert e.value.status == code


def test_create_rejects_bad_buffers():
    cfg = tsdf.tsdf_config(0.01, 0.04, 4096, 0)
    b = _buffers()
    b.weight = None
    with pytest.raises(tsdf.TsdfError) as e:
        tsdf.tsdf_create(cfg, b)
    assert e.value.status == tsdf.TSDF_EINVAL
    b = _buffers()
    b.r = 0x10008
    with pytest.raises(tsdf.TsdfError) as e:
        tsdf.tsdf_create(cfg, b)
    assert e.value.status == tsdf.TSDF_EALIGN
    b = _buffers()
    b.scratch = None                                  # the owner update needs its work list
    with pytest.raises(tsdf.TsdfError) as e:
        tsdf.tsdf_create(cfg, b)
    assert e.value.status == tsdf.TSDF_EINVAL


def test_null_handle_calls():
    f = tsdf.tsdf_frame()
    for fn in (tsdf.tsdf_allocate, tsdf.tsdf_update, tsdf.tsdf_integrate):
        with pytest.raises(tsdf.TsdfError):
            fn(None, f)
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_integrate_batch_noalloc(None, [f])
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_extract_mesh(None, 0, 0, 0)
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_get_stats(None)
    tsdf.tsdf_destroy(None)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="passes made-up device addresses: host-side validation only, "
                                           "never where a kernel could be launched")
def test_microbench_rejects_bad_arguments():
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_mb_copy(0x1000, 0x2000, 17)
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_mb_atomic_add_f32(0x1000, 1000, 10, tsdf.MB_RANDOM)      # not a power of two
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_mb_atomic_add_f32(0x1000, 256, 10, tsdf.MB_BLOCK_ROW)    # under one block
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_mb_cas_u64(0, 1024, 10)
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_mb_lds_atomic(3, tsdf.MB_LDS_RANDOM, 8, 16, 0x1000)       # no such operand type
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_mb_lds_atomic(tsdf.MB_LDS_U32, 4, 8, 16, 0x1000)          # no such pattern
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_mb_lds_atomic(tsdf.MB_LDS_U32, tsdf.MB_LDS_SAME, 8, 16, 0)  # no sink
