"""Host-side pieces of bench.py: the shader-clock reading (rocm-smi's JSON and text forms)
and the FLOP counts behind its metric."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_sclk_from_json(bench):
    text = ('{"card0": {"GPU ID": "0x75a3", "fclk clock speed:": "(2000Mhz)", '
            '"sclk clock speed:": "(1640Mhz)", "sclk clock level:": "S"}}')
    assert bench.parse_sclk_mhz(text) == 1640.0


def test_sclk_first_card_in_order(bench):
    text = ('{"card1": {"sclk clock speed:": "(900Mhz)"}, '
            '"card0": {"sclk clock speed:": "(2100Mhz)"}, "system": "x"}')
    assert bench.parse_sclk_mhz(text) == 2100.0


def test_sclk_from_text(bench):
    text = ("============ ROCm System Management Interface ============\n"
            "GPU[0]\t\t: mclk clock level: 3: (1900Mhz)\n"
            "GPU[0]\t\t: sclk clock level: S: (1982Mhz)\n")
    assert bench.parse_sclk_mhz(text) == 1982.0


def test_sclk_missing(bench):
    assert bench.parse_sclk_mhz("") is None
    assert bench.parse_sclk_mhz('{"card0": {"mclk clock speed:": "(1900Mhz)"}}') is None
    assert bench.parse_sclk_mhz("no GPU found\n") is None


def test_flop_counts(bench):
    # forward 4 B H N^2 d, backward 2.5 times that, both halved under the mask
    assert bench.fwd_flops(4, 8192, 16, 128, False) == 4.0 * 4 * 16 * 8192 ** 2 * 128
    assert bench.bwd_flops(4, 8192, 16, 128, False) == 2.5 * bench.fwd_flops(4, 8192, 16,
                                                                             128, False)
    assert bench.fwd_flops(1, 1024, 12, 64, True) == 0.5 * bench.fwd_flops(1, 1024, 12, 64,
                                                                           False)
    # 4096 FLOP per clock per CU at 2.4 GHz on 256 CUs is the 2.5 PFLOP/s vendor figure
    assert abs(256 * 2.4e9 * bench.BF16_FLOP_PER_CLK_CU / 1e12 - bench.PEAK_BF16_TFLOPS) \
        < 0.01 * bench.PEAK_BF16_TFLOPS


def test_sclk_json_after_warning(bench):
    # rocm-smi may print a warning line before its JSON object
    text = ("WARNING: AMD GPU device(s) is/are in a low-power state. Check power "
            "control/runtime_status\n\n"
            '{"card0": {"mclk clock speed:": "(2000Mhz)", "mclk clock level:": "0", '
            '"sclk clock speed:": "(1814Mhz)", "sclk clock level:": "1"}}\n')
    assert bench.parse_sclk_mhz(text) == 1814.0
    assert bench.parse_sclk_mhz('{"card0": {"sclk clock level": "1 (158Mhz)"}}') == 158.0
