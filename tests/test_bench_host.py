"""bench.py's host-side figures (CPU): the per-block round-trip error summary
and the algorithmic byte counts it reports."""
import numpy as np
import pytest
import torch

import bench


def test_roundtrip_error_stats_on_known_blocks():
    B = 4
    # three blocks: errors 0 / [0.1, 0, 0, 0] / [0.2, 0.2, 0.2, 0.2]; absmax 1, 2, 4
    x = torch.tensor([1.0, 0, 0, 0, 2.0, 0, 0, 0, 4.0, 1, 1, 1])
    y = x.clone()
    y[4] -= 0.1
    y[8:] += 0.2
    st = bench.roundtrip_error_stats(torch, x, y, B)
    assert st["blocks"] == 3
    bm = st["block_max_abs_err"]
    assert np.isclose(bm["max"], 0.2, atol=1e-6) and np.isclose(bm["mean"], (0 + 0.1 + 0.2) / 3, atol=1e-6)
    assert np.isclose(st["block_mean_abs_err"]["max"], 0.2, atol=1e-6)
    assert np.isclose(st["block_max_rel_err"]["max"], 0.05, atol=1e-6)      # 0.1 / 2 and 0.2 / 4
    assert np.isclose(st["block_mean_rel_err"]["mean"], (0 + 0.025 / 2 + 0.2 / 4) / 3, atol=1e-6)


def test_algorithmic_byte_counts():
    assert bench.q8_bytes_per_elem(2048) == 5.0 + 4.0 / 2048                 # one pass
    assert np.isclose(bench.adam_bytes_per_param(), 14.0078125)
    assert np.isclose(bench.w4_bytes_per_weight(), 2.5159, atol=1e-4)
    # the fused 4-bit product at 4096 x 4096, one row of activations: 8.67 MB
    assert np.isclose(bench.dq4_matmul_bytes(1, 4096, 4096) / 1e6, 8.67, atol=0.01)


def test_near_midpoint_mask_counts_one_ulp_on_either_side():
    mids = torch.tensor([-0.25, 0.5], dtype=torch.float64)
    ulps = torch.tensor([np.spacing(np.float32(0.25)), np.spacing(np.float32(0.5))], dtype=torch.float64)
    half = np.float32(0.5)
    vals = np.array([half, np.nextafter(half, np.float32(1)), np.nextafter(half, np.float32(0)),
                     np.float32(0.5 + 2 * 2.0 ** -24), np.float32(-0.25), np.float32(0.0), np.float32(0.9)],
                    dtype=np.float32)
    got = bench._near_midpoint_mask(torch, torch.from_numpy(vals), mids, ulps).numpy()
    assert got.tolist() == [True, True, True, False, True, False, False]


def test_layouts_place_views_as_documented():
    f32, u8 = torch.float32, torch.uint8
    specs = [(5, f32, "p"), (5, u8, "m"), (70, f32, "p"), (70, u8, "m"), (3, f32, "a")]
    a = bench.Layout(torch, "cpu", specs, "arena")
    base = a.buf.data_ptr()
    assert [v.data_ptr() - base for v in a.views] == [i * bench.ARENA_ALIGN for i in range(5)]
    assert [v.numel() for v in a.views] == [5, 5, 70, 70, 3] and [v.dtype for v in a.views] == [f32, u8, f32, u8, f32]
    k = bench.Layout(torch, "cpu", specs, "per-kind")
    base = k.buf.data_ptr()
    offs = [v.data_ptr() - base for v in k.views]
    # regions on 2 MiB boundaries in order of first appearance; a tensor's element offset is the same in each region
    rp, rm, ra = 0, bench.KIND_ALIGN, 2 * bench.KIND_ALIGN
    assert offs == [rp, rm, rp + 64 * 4, rm + 64, ra]
    for v, n in zip(k.views, [5, 5, 70, 70, 3]):
        v.fill_(1)
        assert v.numel() == n and float(v.sum()) == n
    t = bench.Layout(torch, "cpu", specs, "per-tensor")
    assert t.buf is None and [v.numel() for v in t.views] == [5, 5, 70, 70, 3]
    with pytest.raises(ValueError):
        bench.Layout(torch, "cpu", specs, "interleaved")


def _counter_csv(path, rows):
    """A counter_collection.csv as rocprofv3 writes it: one row per dispatch and
    counter instance (Dispatch_Id, Kernel_Name, Counter_Value, ...)."""
    import csv
    path.mkdir(parents=True)
    with open(path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, name, vals in rows:
            for v in vals:                      # instances (XCDs) of one dispatch
                w.writerow([d, name, "C", v])


def test_traffic_summary_scales_counters_by_the_copy(tmp_path):
    ak = "void " + bench.ADAMW_KERNEL + "(qb::TensorDesc, ...)"
    other = "qb::k_dequant<4, 2, true, true, false>"
    # copy calibration: a fill, then five 1 GiB copies reading 512 MiB-worth (fetch) and 1 GiB (write)
    _counter_csv(tmp_path / "cf", [(1, "fill", [0.0])] + [(2 + i, "copy", [262144.0, 262144.0]) for i in range(5)])
    _counter_csv(tmp_path / "cw", [(1, "fill", [1 << 20])] + [(2 + i, "copy", [524288.0, 524288.0]) for i in range(5)])
    # two AdamW dispatches among other kernels, each instance half of the total
    _counter_csv(tmp_path / "bf", [(1, other, [5.0]), (2, ak, [1000.0, 1000.0]), (3, ak, [1100.0, 1100.0])])
    _counter_csv(tmp_path / "bw", [(1, other, [7.0]), (2, ak, [3000.0, 3000.0]), (3, ak, [3000.0, 3000.0])])
    out = tmp_path / "traffic.json"
    bench.traffic_summary(*(str(tmp_path / d) for d in ("bf", "bw", "cf", "cw")), out=str(out))
    import json
    rec = json.load(open(out))
    assert np.isclose(rec["fetch_factor"], 2.0) and np.isclose(rec["write_factor"], 1.0)
    assert np.isclose(rec["fetch_size_kib_per_dispatch"], 2100.0) and rec["dispatches"] == {"fetch": 2, "write": 2}
    assert np.isclose(rec["hbm_bytes_per_launch"], 2100.0 * 1024 * 2 + 6000.0 * 1024)
    assert rec["kernel_sources"] == list(bench.ADAMW_SOURCES)
    assert rec["kernel_source_sha256"] == bench.kernel_source_digest(bench.ADAMW_SOURCES)
    assert np.isclose(rec["algorithmic_bytes_per_launch"], 6_738_415_616 * bench.adam_bytes_per_param())


def test_traffic_digest_covers_only_the_adamw_sources():
    every = bench.kernel_source_digest()
    assert bench.kernel_source_digest(bench.ADAMW_SOURCES) != every
    assert bench.kernel_source_digest(reversed(bench.ADAMW_SOURCES)) == bench.kernel_source_digest(bench.ADAMW_SOURCES)


def test_matmul_weight_rotation_outgrows_the_last_level_cache():
    seen = []
    r = bench.Rotation(3, seen.append)
    for _ in range(7):
        r()
    assert seen == [0, 1, 2, 0, 1, 2, 0]
    for n in (4096 * 4096 // 2, 11008 * 4096 // 2, 3 * 4096 * 4096 // 2, 2 * 11008 * 4096 // 2):
        c = bench.mm_copies(n)
        assert 2 <= c <= bench.MM_MAX_COPIES and c * n >= 2 * (256 << 20)     # twice the cache at least


def test_pattern_tables_pack_descriptors_and_first_tiles():
    # three tensors of 2048, 2049 and 1 elements at block 2048: 1, 2 and 1 tiles
    rows = [((11, 12, 13), 2048), ((21, 22, 23), 2049), ((31, 32, 33), 1)]
    descs, begins, total = bench._pattern_tables(torch, "cpu", rows, 2048)
    assert total == 4
    assert begins.tolist() == [0, 1, 3, 4]
    assert descs.shape == (3, 8) and descs.dtype == torch.int64
    assert descs[1].tolist() == [21, 22, 23, 2049, 0, 0, 0, 0]
    # six pointers (the AdamW descriptor): n in the seventh word, one word of padding
    d6, _, _ = bench._pattern_tables(torch, "cpu", [((1, 2, 3, 4, 5, 6), 7)], 2048)
    assert d6[0].tolist() == [1, 2, 3, 4, 5, 6, 7, 0]
