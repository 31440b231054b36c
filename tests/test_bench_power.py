"""The benchmark's power phase on the host: the reduction of the driver's
energy-counter readings to an average socket power, and the phase's loop
against a stand-in for the amdsmi module and torch's device calls (no GPU)."""
import bench

RES_UJ = 15.3  # counter resolution in microjoules, as the driver reports it


def _counts(joules):
    return round(joules / (RES_UJ * 1e-6))


def test_constant_power_over_whole_windows():
    # 1,390 W for three one-second windows, then 1,400 W for one
    e = [0, _counts(1390), _counts(2780), _counts(4170), _counts(5570)]
    ts = [10**9 * (5 + k) for k in range(5)]
    clk = [[1650 + x for x in range(8)]] * 5
    r = bench.power_from_readings(list(zip(ts, e, [RES_UJ] * 5, clk)), cap_w=1400.0)
    assert abs(r["avg_w"] - 5570 / 4) < 0.5
    assert abs(r["window_w_min"] - 1390) < 0.5 and abs(r["window_w_max"] - 1400) < 0.5
    assert r["windows"] == 4 and abs(r["seconds"] - 4.0) < 1e-9
    assert r["cap_w"] == 1400.0
    assert r["gfxclk_mhz_per_xcd"] == [1650.0 + x for x in range(8)]
    assert r["gfxclk_mhz_mean"] == 1653.5


def test_uneven_windows_weigh_by_time():
    # 0.5 s at 1,000 W then 1.5 s at 1,400 W: 1,300 W on average
    ts = [0, 5 * 10**8, 2 * 10**9]
    e = [0, _counts(500), _counts(500 + 2100)]
    r = bench.power_from_readings([(t, x, RES_UJ, []) for t, x in zip(ts, e)])
    assert abs(r["avg_w"] - 1300) < 0.5
    assert r["gfxclk_mhz_per_xcd"] is None and r["gfxclk_mhz_mean"] is None


def test_clocks_come_from_the_windows_inside_the_load():
    # the first reading's clocks describe the window before the first update
    ts = [0, 10**9, 2 * 10**9]
    clk = [[100] * 8, [1600] * 8, [1700] * 8]
    r = bench.power_from_readings([(t, _counts(1400) * k, RES_UJ, c)
                                   for k, (t, c) in enumerate(zip(ts, clk))])
    assert r["gfxclk_mhz_per_xcd"] == [1650.0] * 8


def test_too_few_readings():
    assert bench.power_from_readings([]) is None
    assert bench.power_from_readings([(0, 0, RES_UJ, [])]) is None
    assert bench.power_from_readings([(5, 0, RES_UJ, []), (5, 10, RES_UJ, [])]) is None


def test_power_phase_off():
    assert bench.measure_power(lambda i: None, None, 0) is None


class _FakeSmi:
    """Stands in for the amdsmi module: one device whose energy counter
    advances by `watts` joules per update, each call being one update one
    second after the last."""

    def __init__(self, watts=1400.0, fail_energy=False):
        self.watts, self.fail_energy = watts, fail_energy
        self.ts, self.count, self.shut = 10**12, 0, False

    def amdsmi_init(self):
        pass

    def amdsmi_shut_down(self):
        self.shut = True

    def amdsmi_get_processor_handles(self):
        return ["h0"]

    def amdsmi_get_gpu_device_bdf(self, h):
        return "0000:8b:00.0"

    def amdsmi_get_power_cap_info(self, h):
        return {"power_cap": 1_400_000_000}

    def amdsmi_get_energy_count(self, h):
        if self.fail_energy:
            raise RuntimeError("no energy counter")
        self.ts += 10**9
        self.count += round(self.watts / (RES_UJ * 1e-6))
        return {"energy_accumulator": self.count, "counter_resolution": RES_UJ,
                "timestamp": self.ts}

    def amdsmi_get_gpu_metrics_info(self, h):
        return {"current_gfxclks": [1700, 1620] * 4}


def _fake_torch_cuda(monkeypatch):
    import torch

    class Prop:
        pci_domain_id, pci_bus_id, pci_device_id = 0, 0x8B, 0

    class Event:
        def record(self):
            pass

        def synchronize(self):
            pass

    monkeypatch.setattr(torch.cuda, "get_device_properties", lambda dev: Prop())
    monkeypatch.setattr(torch.cuda, "Event", Event)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)


def test_power_phase_loop_with_a_fake_driver(monkeypatch):
    import sys
    smi = _FakeSmi(1400.0)
    monkeypatch.setitem(sys.modules, "amdsmi", smi)
    _fake_torch_cuda(monkeypatch)
    steps = []
    r = bench.measure_power(steps.append, None, 0.15)
    assert steps and steps == list(range(len(steps)))  # the step ran back to back
    assert r is not None and abs(r["avg_w"] - 1400.0) < 0.5 and r["windows"] >= 2
    assert r["cap_w"] == 1400.0 and r["gfxclk_mhz_per_xcd"] == [1700.0, 1620.0] * 4
    assert smi.shut


def test_power_phase_gives_up_quietly_when_the_driver_fails(monkeypatch):
    import sys
    smi = _FakeSmi(fail_energy=True)
    monkeypatch.setitem(sys.modules, "amdsmi", smi)
    _fake_torch_cuda(monkeypatch)
    assert bench.measure_power(lambda i: None, None, 0.1) is None
    assert smi.shut
    other = _FakeSmi()
    other.amdsmi_get_gpu_device_bdf = lambda h: "0000:01:00.0"  # not this device
    monkeypatch.setitem(sys.modules, "amdsmi", other)
    assert bench.measure_power(lambda i: None, None, 0.1) is None
