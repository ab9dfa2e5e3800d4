"""Host logic of bench.py that feeds the reported roofline (CPU only, no GPU work).

The HBM traffic of a GEMM launch comes from two rocprofv3 counter passes (FETCH_SIZE, then
WRITE_SIZE, in KiB per dispatch, one row per hardware instance). Each counter is scaled by what
it reads for a plain 1 GiB device copy in the same run, and the resident-grid GEMM launches are
told apart by their order in the step (Fprop, Dgrad, Wgrad). These tests feed synthetic counter
files with known answers through that code.
"""
import csv
import json

import pytest

import bench

T, K, N = 16384, 28672, 8192          # the 70B down-projection: tokens, FFN, hidden
SHAPES = {"fprop": (T, N, K), "dgrad": (T, K, N), "wgrad": (N, K, T)}  # (M, N, K) per GEMM
GEMM = "(anonymous namespace)::gemm_mx_stream_kernel<4, 4, 2, 8, 8, 1, false, 4, 4>(args)"
QOUT = "(anonymous namespace)::gemm_mx_stream_kernel<4, 4, 2, 8, 8, 1, true, 4, 4>(args)"
FP8 = "(anonymous namespace)::gemm_mx_stream_kernel<4, 4, 2, 16, 2, 0, false, 0, 0>(args)"
QUANT = "(anonymous namespace)::quant_rows_kernel<true, true, true, true>(args)"
PP = "void (anonymous namespace)::gemm_mx_pp_kernel<4, 4, false>(unsigned char const*, int)"
PP_FP8 = "void (anonymous namespace)::gemm_mx_pp_kernel<1, 0, false>(unsigned char const*, int)"
PP_QOUT = "void (anonymous namespace)::gemm_mx_pp_kernel<4, 4, true>(unsigned char const*, int)"
COPY = "__amd_rocclr_copyBuffer"
FETCH_KIB = {"fprop": 1_400_000.0, "dgrad": 1_500_000.0, "wgrad": 1_450_000.0}


def out_kib(name):
    M, Nn, _ = SHAPES[name]
    return 2 * M * Nn / 1024.0      # bf16 output, write factor 1


def write_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, total value); each value is split over 4 instances."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, name, value in rows:
            for part in (0.1, 0.2, 0.3, 0.4):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": value * part})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": "OTHER",
                        "Counter_Value": 1e12})


def dispatches(value_of, copy_kib, steps=3, write_scale=None, gemm=GEMM, extra=()):
    """A run in dispatch order: per step, a quantizer and the three GEMMs; then the quantizing
    epilogue and an MXFP8 GEMM (not the plain MXFP4 kernel), `extra` launches, then the
    calibration copy."""
    rows, d = [], 1
    for _ in range(steps):
        rows.append((d, QUANT, 123.0)); d += 1
        for name in bench.TRAFFIC_ORDER:
            v = value_of(name)
            if write_scale and name in write_scale:
                v *= write_scale[name]
            rows.append((d, gemm, v)); d += 1
    rows += [(d, QOUT, 9e9), (d + 1, FP8, 9e9)]
    d += 2
    for name in extra:
        rows.append((d, name, 7e9)); d += 1
    rows += [(d, COPY, copy_kib), (d + 1, COPY, 10.0)]
    return rows


@pytest.fixture
def record_path(tmp_path, monkeypatch):
    p = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    return p


def make_files(tmp_path, write_scale=None, **kw):
    fetch_csv, wr_csv = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the copy reads 1 GiB but FETCH_SIZE reports half of it (factor 2); WRITE_SIZE reports all
    write_csv(fetch_csv, "FETCH_SIZE", dispatches(lambda n: FETCH_KIB[n], (1 << 30) / 2048.0, **kw))
    write_csv(wr_csv, "WRITE_SIZE", dispatches(out_kib, (1 << 30) / 1024.0,
                                               write_scale=write_scale, **kw))
    return str(fetch_csv), str(wr_csv)


def test_counter_values_sums_instances_in_dispatch_order(tmp_path):
    p = tmp_path / "c.csv"
    write_csv(p, "FETCH_SIZE", [(7, GEMM, 30.0), (2, GEMM, 10.0), (5, COPY, 4.0), (3, GEMM, 20.0)])
    vals = bench.counter_values(str(p), "FETCH_SIZE")
    assert vals[GEMM] == pytest.approx([10.0, 20.0, 30.0])
    assert vals[COPY] == pytest.approx([4.0])


@pytest.mark.parametrize("kw", [{}, {"gemm": PP}, {"gemm": PP, "extra": (GEMM,) * 12},
                                {"gemm": PP, "extra": (PP_FP8, PP_QOUT) * 6}],
                         ids=["stream", "pingpong", "pingpong_then_stream",
                              "pingpong_then_fp8_and_quantizing"])
def test_write_traffic_record(tmp_path, record_path, monkeypatch, kw):
    # the ping-pong kernel's launches are the step's when present, whatever streaming-kernel
    # launches follow in the run
    fetch_csv, wr_csv = make_files(tmp_path, **kw)
    monkeypatch.setattr(bench, "sha", lambda path: "0123456789abcdef")
    bench.write_traffic(fetch_csv, wr_csv, "llama70b_down")
    rec = json.load(open(record_path))
    assert rec["gemm_sha"] == "0123456789abcdef"
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    for name, (M, Nn, Kk) in SHAPES.items():
        # fetch: KiB x 1024 x 2; write: exactly the bf16 output
        want = FETCH_KIB[name] * 1024 * 2 + 2 * M * Nn
        assert rec[f"{name}_hbm_bytes_per_launch"] == pytest.approx(want, rel=1e-12)
        # packed E2M1 codes (K/2 bytes per row) and one scale byte per 32 of both operands,
        # plus the bf16 output
        codes = (M * Kk + Nn * Kk) // 2
        scales = (M * Kk + Nn * Kk) // 32
        assert rec[f"{name}_algorithmic_bytes_per_launch"] == codes + scales + 2 * M * Nn


def test_load_traffic_checks_kernel_hash(tmp_path, record_path, monkeypatch):
    fetch_csv, wr_csv = make_files(tmp_path)
    monkeypatch.setattr(bench, "sha", lambda path: "aaaa")
    bench.write_traffic(fetch_csv, wr_csv, "llama70b_down")
    key = "wgrad_hbm_bytes_per_launch"
    assert bench.load_traffic(key, "llama70b_down") == json.load(open(record_path))[key]
    assert bench.load_traffic(key, "llama8b_up") is None
    monkeypatch.setattr(bench, "sha", lambda path: "bbbb")  # the kernel changed since
    assert bench.load_traffic(key, "llama70b_down") is None


def test_write_traffic_rejects_a_launch_that_is_not_its_gemm(tmp_path, record_path):
    # Dgrad writing 20% more than its output means the order-based labels are off
    fetch_csv, wr_csv = make_files(tmp_path, write_scale={"dgrad": 1.2})
    with pytest.raises(SystemExit, match="dgrad"):
        bench.write_traffic(fetch_csv, wr_csv, "llama70b_down")
    assert not record_path.exists()


def test_write_traffic_needs_the_calibration_copy(tmp_path, record_path):
    fetch_csv, wr_csv = make_files(tmp_path)
    rows = [r for r in csv.DictReader(open(fetch_csv)) if r["Kernel_Name"] != COPY]
    with open(fetch_csv, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)
    with pytest.raises(SystemExit, match="copy"):
        bench.write_traffic(fetch_csv, wr_csv, "llama70b_down")


def test_write_traffic_other_workload(tmp_path, record_path):
    fetch_csv, wr_csv = make_files(tmp_path)
    with pytest.raises(SystemExit):
        bench.write_traffic(fetch_csv, wr_csv, "llama8b_up")


def test_cpu_baseline_on_a_small_layer():
    """The CPU baseline runs the oracle as it stands on a host-side stand-in for the layer and
    reports the pieces its whole-step figure is built from."""
    import torch
    T, K, N = 256, 1024, 128
    g = torch.Generator().manual_seed(0)

    class Small:
        pass
    L = Small()
    L.T, L.K, L.N = T, K, N
    L.X = torch.randn((T, K), generator=g).to(torch.bfloat16)
    L.W = torch.randn((N, K), generator=g).to(torch.bfloat16)
    L.dY = torch.randn((T, N), generator=g).to(torch.bfloat16)
    L.fprop_q = L.dgrad_q = L.wgrad_q = (1, 0x1234, 1, 1)
    L.seeds = {"X": 1, "W": 2, "dY": 3}
    L.alpha = {"fprop": -5, "dgrad": -5, "wgrad": -5}
    L.flops = {"fprop": 2.0 * T * N * K, "dgrad": 2.0 * T * K * N, "wgrad": 2.0 * N * K * T}
    u8 = lambda *s: torch.randint(0, 256, s, generator=g, dtype=torch.uint8)  # noqa: E731
    sc = lambda *s: torch.randint(120, 134, s, generator=g, dtype=torch.uint8)  # noqa: E731
    L.buf = {"Xq": (u8(T, K // 2), sc(T, K // 32)), "Wq": (u8(N, K // 2), sc(N, K // 32)),
             "dYq": (u8(T, N // 2), sc(T, N // 32)), "Wt": (u8(K, N // 2), sc(K, N // 32)),
             "dYt": (u8(N, T // 2), sc(N, T // 32)), "Xt": (u8(K, T // 2), sc(K, T // 32))}
    cb = bench.cpu_baseline(L, gemm_rows=8, gemm_elements=16)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert cb["cores"] == bench.cpu_threads()
    assert set(cb["quantize"]) == {"Xq", "Wq", "dYq", "Wt", "dYt", "Xt"}
    assert cb["quantize"]["Xq"]["elements"] == T * K
    for name in ("fprop", "dgrad", "wgrad"):
        gm = cb["gemm"][name]
        assert gm["sample_rows"] == 8 and gm["matmul_GFLOP_per_s"] > 0
        assert gm["full_gemm_extrapolated_s"] > 0
    json.dumps(cb)
