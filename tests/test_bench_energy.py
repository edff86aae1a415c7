"""Host logic of bench.py's energy measurement, with stand-ins for amdsmi and
torch: joules from the accumulator difference, the PCI-bus device match, and
the error records when amdsmi is missing or no device matches."""
import sys
import time
import types

import pytest

import bench


class FakeTorch:
    class cuda:
        bus = 0x75

        @staticmethod
        def synchronize():
            pass

        @classmethod
        def get_device_properties(cls, i):
            return types.SimpleNamespace(pci_bus_id=cls.bus)


def fake_amdsmi(buses, uj_per_launch, resolution=15.3):
    m = types.ModuleType("amdsmi")
    state = {"launches": 0, "shut": False}
    m.AmdSmiClkType = types.SimpleNamespace(GFX=1)
    m.amdsmi_init = lambda: None
    m.amdsmi_get_processor_handles = lambda: list(range(len(buses)))
    m.amdsmi_get_gpu_device_bdf = lambda h: "0000:%02x:00.0" % buses[h]
    m.amdsmi_get_energy_count = lambda h: {
        "energy_accumulator": int(state["launches"] * uj_per_launch / resolution),
        "counter_resolution": resolution, "timestamp": time.perf_counter_ns()}
    m.amdsmi_get_power_info = lambda h: {"current_socket_power": 1000, "power_limit": "N/A"}
    m.amdsmi_get_clock_info = lambda h, t: {"clk": 2100}

    def shut():
        state["shut"] = True
    m.amdsmi_shut_down = shut
    return m, state


@pytest.fixture
def with_amdsmi(monkeypatch):
    def install(*a, **kw):
        m, state = fake_amdsmi(*a, **kw)
        monkeypatch.setitem(sys.modules, "amdsmi", m)
        return state
    return install


def test_energy_from_accumulator(with_amdsmi):
    state = with_amdsmi([0x05, 0x75, 0x15], uj_per_launch=2e6)   # 2 J per launch

    def step():
        state["launches"] += 1
        time.sleep(0.001)
    flops = 4e12
    r = bench.energy_run(step, flops, FakeTorch, seconds=0.0)
    n = r["launches"]
    assert n == 10                                  # the minimum loop
    assert r["joules"] == pytest.approx(2.0 * n, rel=1e-3)
    # power from the counter's own timestamps (here host nanoseconds)
    assert r["counter_window_s"] == pytest.approx(r["seconds"], rel=5e-2)
    assert r["TFLOP/J"] == pytest.approx(flops / 2.0 / 1e12, rel=5e-2)
    assert r["socket_watts_sampled_median"] is None or r["socket_watts_sampled_median"] == 1000
    assert state["shut"]


def test_energy_no_matching_device(with_amdsmi):
    state = with_amdsmi([0x05, 0x15], uj_per_launch=1.0)
    r = bench.energy_run(lambda: None, 1.0, FakeTorch, seconds=0.0)
    assert "error" in r and "0x75" in r["error"]
    assert state["shut"]


def test_energy_without_amdsmi(monkeypatch):
    monkeypatch.setitem(sys.modules, "amdsmi", None)    # import raises ImportError
    r = bench.energy_run(lambda: None, 1.0, FakeTorch, seconds=0.0)
    assert r["error"].startswith("amdsmi not importable")
