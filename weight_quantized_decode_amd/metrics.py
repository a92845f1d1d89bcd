"""Byte-model arithmetic used by the bench report.

The pages estimate decode speed from the bytes one token must read: bytes per token divided by
memory bandwidth is the minimum read time, and its reciprocal an upper bound on tokens per
second; conversely tokens per second times bytes per token is the effective bandwidth
("Making a ternary reasoning model fast in vLLM", "A rough speed limit" and the 17% estimate
under "Reading the prompt and writing the answer"; trapetum "Benchmarks", the Llama-2-70B 2-bit
section, "about 670 GB/s, two thirds of the card's 1,008 GB/s").
"""
from __future__ import annotations

MI355X_HBM_PEAK_GBPS = 8000.0  # published HBM3E peak, GB/s (1 GB = 1e9 bytes)


def floor_seconds(bytes_per_token: float, bandwidth_gbps: float) -> float:
    """Minimum time to stream the bytes of one token at the given bandwidth."""
    return bytes_per_token / (bandwidth_gbps * 1e9)


def ceiling_tok_s(bytes_per_token: float, bandwidth_gbps: float) -> float:
    return 1.0 / floor_seconds(bytes_per_token, bandwidth_gbps)


def effective_gbps(tok_s: float, bytes_per_token: float) -> float:
    return tok_s * bytes_per_token / 1e9


def gbps(bytes_moved: float, seconds: float) -> float:
    return bytes_moved / seconds / 1e9


def fraction_of_peak(achieved_gbps: float, peak_gbps: float = MI355X_HBM_PEAK_GBPS) -> float:
    return achieved_gbps / peak_gbps


def bits_per_weight(nbytes: int, nweights: int) -> float:
    return nbytes * 8.0 / nweights
