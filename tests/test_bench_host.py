"""Host logic of bench.py, on the CPU: which kernel the roofline and traffic
figures describe, the traffic record's key on the kernel sources, the PMC
summary's calibration arithmetic, and the decode workload's algorithmic
bytes against the EP blog's per-expert figure (section 6.3: 88 MB per
expert = 3 matrices of 7168 x 2048 fp16)."""
import json
import os

import numpy as np
import pytest
import torch

import bench
import moe_synth

# kernel names as rocprofv3 prints them (PMC runs: mangled; kernel traces:
# demangled); template arguments <weight, x, subtiles, epilogue, K waves,
# chunks, fragment layout> and <tile rows, matrices, epilogue, gathered,
# fragment layout, combine in the tail>, epilogue 1 = SwiGLU
STREAM = ("_ZN3moe12_GLOBAL__N_118stream_gemm_kernelIDF16_Li1ELi4ELi{}ELi4ELi2ELb1EEEv"
          "NS_10StreamArgsE")
STREAM_F32 = ("void moe::(anonymous namespace)::stream_gemm_kernel<float, 1, 4, {}, 4, 2, false>"
              "(moe::StreamArgs)")
TILED = "void moe::(anonymous namespace)::tiled_gemm_kernel<{}>(moe::StreamArgs, int, int)"
TILED_MANGLED = ("_ZN3moe12_GLOBAL__N_117tiled_gemm_kernelILi256ELi2ELi1ELb{}ELb1ELb0EEEv"
                 "NS_10StreamArgsEii")
COPY = ("void at::native::vectorized_elementwise_kernel<8, at::native::AUnaryFunctor<c10::Half, "
        "c10::Half, c10::Half, at::native::binary_internal::MulFunctor<float> >>(int)")


def test_dominant_kernel_is_the_swiglu_gate_up_launch():
    assert bench.is_dominant(STREAM.format(1), "stream")
    assert bench.is_dominant(STREAM_F32.format(1), "stream")
    for epi in (0, 2):  # down projection, router logits
        assert not bench.is_dominant(STREAM.format(epi), "stream")
        assert not bench.is_dominant(STREAM_F32.format(epi), "stream")
    assert bench.is_dominant(TILED.format("256, 2, 1, true, true, false"), "tiled")
    assert bench.is_dominant(TILED.format("256, 2, 1, true, false, false"), "tiled")
    assert bench.is_dominant(TILED_MANGLED.format(1), "tiled")
    for args in ("256, 1, 0, false, true, false", "256, 1, 0, false, true, true",
                 "128, 1, 2, false, false, false", "256, 2, 1, false, true, false"):
        assert not bench.is_dominant(TILED.format(args), "tiled")
    assert not bench.is_dominant(TILED_MANGLED.format(0), "tiled")
    # one kind never matches the other's kernels
    assert not bench.is_dominant(STREAM.format(1), "tiled")
    assert not bench.is_dominant(TILED.format("256, 2, 1, true, true, false"), "stream")
    assert bench.dominant_kind(4) == "tiled"
    assert all(bench.dominant_kind(n) == "stream" for n in (1, 2, 3, 5))


def test_kernel_labels():
    assert bench.kernel_label(TILED.format("256, 2, 1, true, true, false")) == \
        "tiled_gemm_kernel gate/up (256-row tiles)"
    assert bench.kernel_label(TILED.format("256, 1, 0, false, true, false")) == \
        "tiled_gemm_kernel down (256-row tiles)"
    assert bench.kernel_label(TILED.format("256, 1, 0, false, true, true")) == \
        "tiled_gemm_kernel down (256-row tiles) + combine in the tail"
    assert bench.kernel_label("_ZN3moe12_GLOBAL__N_117tiled_gemm_kernelILi256ELi1ELi0ELb0ELb1ELb1EEEv"
                              "NS_10StreamArgsEii").endswith("combine in the tail")
    assert bench.kernel_label(TILED.format("128, 1, 2, false, false, false")) == \
        "tiled_gemm_kernel router (128-row tiles)"
    assert bench.kernel_label(STREAM.format(1)) == "stream_gemm_kernel gate/up"


def test_traffic_record_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    rec = tmp_path / "rec.json"
    monkeypatch.setattr(bench, "traffic_path", lambda kind, workload: str(rec))
    assert bench.load_traffic("tiled", "w") is None  # no record
    rec.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash("tiled"),
                               "traffic_bytes_per_launch": 1234.5}))
    assert bench.load_traffic("tiled", "w") == 1234.5
    # the same record against the other kernel's sources: dropped
    assert bench.kernel_source_hash("stream") != bench.kernel_source_hash("tiled")
    assert bench.load_traffic("stream", "w") is None


def _counter_csv(path, rows):
    path.mkdir(parents=True)
    with open(path / "run_counter_collection.csv", "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for name, counter, value in rows:
            f.write(f'"{name}","{counter}",{value}\n')


def test_pmc_summary_scales_each_counter_by_the_calibration_copy(tmp_path, monkeypatch):
    """A 1 GiB copy reads 1 GiB and writes 1 GiB; whatever a counter reads
    for it fixes that counter's scale (here FETCH reads half, WRITE all)."""
    gib = 1 << 30
    dom = TILED.format("256, 2, 1, true, true")
    other = TILED.format("256, 1, 0, false, true")
    _counter_csv(tmp_path / "fetch", [
        (dom, "FETCH_SIZE", 1000.0), (dom, "FETCH_SIZE", 1004.0), (dom, "FETCH_SIZE", 990.0),
        (other, "FETCH_SIZE", 9.0e6), (COPY, "FETCH_SIZE", gib / 1024 / 2)])
    _counter_csv(tmp_path / "write", [
        (dom, "WRITE_SIZE", 10.0), (dom, "WRITE_SIZE", 12.0), (dom, "WRITE_SIZE", 11.0),
        (other, "WRITE_SIZE", 7.0e6), (COPY, "WRITE_SIZE", gib / 1024)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda kind, workload: str(out))
    bench.summarize_pmc(str(tmp_path / "fetch"), str(tmp_path / "write"), "w", gib, "tiled")
    rec = json.loads(out.read_text())
    assert rec["kernel_source_hash"] == bench.kernel_source_hash("tiled")
    assert rec["counters"]["FETCH_SIZE"]["copy_factor"] == pytest.approx(2.0)
    assert rec["counters"]["WRITE_SIZE"]["copy_factor"] == pytest.approx(1.0)
    # medians of the dominant launches, in bytes
    assert rec["traffic_bytes_per_launch"] == pytest.approx(1000.0 * 1024 * 2 + 11.0 * 1024)


def test_decode_bytes_follow_the_pages_per_expert_figure():
    cfg = moe_synth.config(2)  # EP = 8 rank share, T = 256, 32 local slots
    per_expert = 3 * 7168 * 2048 * 2  # EP blog section 6.3: 88 MB per expert
    assert per_expert == 88_080_384
    counts = np.full(32, 8, np.int32)  # every slot touched, P = 256
    work = bench.algorithmic_work(cfg, counts)
    T, H, P = cfg.T, cfg.H, 256
    assert (work["P"], work["touched"]) == (P, 32)
    vec = T * H * 2  # one [256, 7168] fp16 array: router weights, h, output
    # the layer: every touched expert once, router weights, h and the
    # output; the expert-output round trip and the routing outputs are time
    assert work["layer_bytes"] == 32 * per_expert + 3 * vec == 2_829_582_336
    # gate/up launch: two of the three matrices per touched expert, the
    # gathered rows and the SwiGLU output
    assert work["up"]["bytes"] == 32 * per_expert * 2 // 3 + P * H * 2 + P * cfg.I * 2
    assert work["up"]["flops"] == 2 * 2 * P * H * cfg.I


def test_full_layer_bytes_count_the_touched_and_shared_experts():
    """Whole layer at decode (T = 128, 256 experts, 2 shared): touched
    experts + the shared experts (section 2.1: 176 MB for two) + router +
    h + out.  The shared experts ride in the routed gate/up launch."""
    cfg = moe_synth.config(3)
    counts = np.zeros(256, np.int32)
    counts[:238] = 4
    counts[0] += 1024 - 4 * 238  # P = T * K = 1024 over 238 touched experts
    work = bench.algorithmic_work(cfg, counts)
    assert work["touched"] == 238 and work["P"] == 1024
    assert work["layer_bytes"] == 238 * 88_080_384 + 176_160_768 + 3_670_016 + 2 * 1_835_008
    assert bench.shared_in_routed_launch(cfg)
    H, I, T = cfg.H, cfg.I, cfg.T
    assert work["up"]["bytes"] == ((238 + 2) * 2 * I * H * 2 + (1024 + 2 * T) * (H + I) * 2)


def test_replica_fp8_bytes_follow_the_survey_figure():
    """Imbalanced decode with one replica slot and fp8 rows: 33 touched
    slots; the layer figure is 33 experts + router + h + out, and the
    gate/up launch reads one byte per element of each fp8 row plus its
    fp32 scale."""
    cfg = moe_synth.config(5)
    counts = np.full(33, 16, np.int32)
    work = bench.algorithmic_work(cfg, counts)
    assert work["layer_bytes"] == 2_925_002_752
    P, H, I = 33 * 16, cfg.H, cfg.I
    assert not bench.shared_in_routed_launch(cfg)
    assert work["up"]["bytes"] == 33 * 2 * I * H * 2 + P * (H + 4) + P * I * 2


def test_cpu_baseline_runs_single_and_multi_threaded():
    """The oracle baseline leg on the tiny workload's host inputs: one
    thread first, then several threads on disjoint token blocks."""
    import oracle
    cfg = moe_synth.config(1)
    rep_off, rep_slot, slot_experts = oracle.placement(cfg.E, 1, 0)
    ctx = dict(cfg=cfg, rep=None, h=moe_synth.gen_hidden(cfg), wr=moe_synth.gen_router(cfg),
               bias=moe_synth.gen_router_bias(cfg), shared=moe_synth.gen_shared_weights(cfg),
               host_experts={int(e): moe_synth.gen_expert(cfg, int(e)) for e in slot_experts})
    rec = bench.cpu_baseline(ctx, budget_s=0.3)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["value"] > 0 and rec["single_thread"]["value"] > 0
    assert 1 <= rec["cores"] <= 16 and rec["single_thread"]["cores"] == 1
    assert rec["cpu_model"]


def test_kernel_labels_name_each_layer_kernel():
    assert bench.kernel_label(STREAM.format(1)) == "stream_gemm_kernel gate/up"
    assert bench.kernel_label(STREAM.format(0)) == "stream_gemm_kernel down"
    assert bench.kernel_label(STREAM_F32.format(2)) == "stream_gemm_kernel router"
    assert bench.kernel_label(TILED.format("256, 2, 1, true, true")) == \
        "tiled_gemm_kernel gate/up (256-row tiles)"
    assert bench.kernel_label(TILED_MANGLED.format(0).replace("Li2ELi1", "Li1ELi0")) == \
        "tiled_gemm_kernel down (256-row tiles)"
    assert bench.kernel_label("void moe::(anonymous namespace)::topk_kernel<4, 14>(float const*)") \
        == "topk_kernel"
    assert bench.kernel_label(COPY) == ""


def test_pmc_summary_of_every_kernel(tmp_path, monkeypatch):
    gib = 1 << 30
    up, down = TILED.format("256, 2, 1, true, true"), TILED.format("256, 1, 0, false, true")
    _counter_csv(tmp_path / "fetch", [(up, "FETCH_SIZE", 100.0), (up, "FETCH_SIZE", 104.0),
                                      (down, "FETCH_SIZE", 50.0), (COPY, "FETCH_SIZE", gib / 2048)])
    _counter_csv(tmp_path / "write", [(up, "WRITE_SIZE", 3.0), (down, "WRITE_SIZE", 7.0),
                                      (COPY, "WRITE_SIZE", gib / 1024)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    bench.summarize_pmc_all(str(tmp_path / "fetch"), str(tmp_path / "write"), "w", gib)
    rec = json.loads((tmp_path / "profiles" / "traffic_layer_kernels_w.json").read_text())
    k = rec["kernels"]
    assert k["tiled_gemm_kernel gate/up (256-row tiles)"]["FETCH_SIZE_bytes"] == \
        pytest.approx(102.0 * 1024 * 2)
    assert k["tiled_gemm_kernel down (256-row tiles)"]["WRITE_SIZE_bytes"] == pytest.approx(7 * 1024)


def test_trace_summary_splits_the_prefill_leg(tmp_path):
    """Kernel-trace rows of one benchmark run: the main workload's kernels,
    then the prefill leg from the first LDS-tiled GEMM on; grouped by
    kernel and grid."""
    d = tmp_path / "trace"
    d.mkdir()
    cols = "Kernel_Name,Start_Timestamp,End_Timestamp,Workgroup_Size_X,Grid_Size_X,Grid_Size_Y,Grid_Size_Z"
    rows = [(STREAM.format(1), 0, 2000, 256, 256 * 32, 258, 1),
            (STREAM.format(1), 5000, 7000, 256, 256 * 32, 258, 1),
            (STREAM.format(1), 8000, 8100, 256, 256 * 32, 2, 2),
            (TILED.format("128, 1, 2, false, false"), 10000, 10080, 512, 512 * 256, 1, 1),
            (TILED.format("256, 2, 1, true, true"), 11000, 12000, 512, 512 * 256, 1, 1)]
    with open(d / "run_kernel_trace.csv", "w") as f:
        f.write(cols + "\n")
        for r in rows:
            f.write('"' + r[0] + '",' + ",".join(str(v) for v in r[1:]) + "\n")
    out = bench.summarize_trace(str(d))
    main = {(k["kernel"], tuple(k["grid"])): k for k in out["main"]}
    assert main[("stream_gemm_kernel gate/up", (32, 258, 1))]["calls"] == 2
    assert main[("stream_gemm_kernel gate/up", (32, 258, 1))]["avg_us"] == 2.0
    assert ("stream_gemm_kernel gate/up", (32, 2, 2)) in main
    pre = [k["kernel"] for k in out["prefill"]]
    assert pre == ["tiled_gemm_kernel gate/up (256-row tiles)", "tiled_gemm_kernel router (128-row tiles)"]


def test_step_percentiles_nearest_rank():
    p = bench.percentiles([float(v) for v in range(10, 0, -1)])  # order does not matter
    assert p == {"median": 5.5, "p10": 2.0, "p90": 9.0, "n": 10}
    assert bench.percentiles([3.0]) == {"median": 3.0, "p10": 3.0, "p90": 3.0, "n": 1}
    q = bench.percentiles([1.0, 100.0, 2.0])
    assert q["p10"] == 1.0 and q["p90"] == 100.0 and q["median"] == 2.0


def test_summarize_counters_groups_by_kernel_and_counter(tmp_path):
    d = tmp_path / "pmc" / "host"
    d.mkdir(parents=True)
    rows = [("Kernel_Name", "Counter_Name", "Counter_Value")]
    gate = TILED.format("256, 2, 1, true, true, false")
    down = TILED.format("256, 1, 0, false, true, false")
    for v in (10.0, 30.0, 20.0):
        rows.append((gate, "MfmaFlopsF16", v))
    rows.append((down, "MfmaFlopsF16", 5.0))
    rows.append((down, "MfmaUtil", 40.0))
    rows.append(("some_other_kernel", "MfmaFlopsF16", 99.0))
    with open(d / "run_counter_collection.csv", "w") as f:
        for r in rows:
            f.write(",".join(f'"{x}"' for x in r) + "\n")
    out = bench.summarize_counters(str(tmp_path / "pmc"))
    g = out["tiled_gemm_kernel gate/up (256-row tiles)"]["MfmaFlopsF16"]
    assert g == {"median_per_launch": 20.0, "launches": 3}
    assert out["tiled_gemm_kernel down (256-row tiles)"]["MfmaUtil"]["median_per_launch"] == 40.0
    assert all("other" not in k for k in out)


def test_read_probe_library_validates_before_launch():
    """libmoe_probe.so (built by build()): bad arguments return -1 and
    launch nothing (no device needed)."""
    import ctypes
    path = os.path.join(bench.ROOT, "expert_router_gemm_amd", "libmoe_probe.so")
    if not os.path.exists(path):
        pytest.skip("libmoe_probe.so not built")
    fn = ctypes.CDLL(path).moe_probe_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    fake = 0x100000
    good = dict(buf=fake, nbytes=1 << 20, slab=1 << 16, blocks=4, unroll=8, out=fake)
    for bad in (dict(buf=None), dict(out=None), dict(blocks=0), dict(unroll=3), dict(slab=1000),
                dict(slab=3 << 10), dict(nbytes=(1 << 20) + 1024)):
        a = dict(good, **bad)
        assert fn(a["buf"], a["nbytes"], a["slab"], a["blocks"], a["unroll"], a["out"], None) == -1
