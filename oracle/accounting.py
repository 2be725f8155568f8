"""KV-cache byte and page accounting (oracle; test infrastructure only).

«Servicio…presupuesto de memoria» §3 ("El presupuesto de claves y valores…"): uncompressed K/V state
costs two (K and V) times layers times KV heads times head dimension times
bytes per scalar, per retained token, summed over all retained tokens.
«¿Cuánta memoria reservar para la caché KV?» ("Plantear la fórmula y sus unidades"): the same product with the
symbols L, Hkv, D, q; for unequal lengths the batch-times-length product is
replaced by the sum of stored positions; GiB = 2**30 bytes, GB = 10**9.
«Servicio…presupuesto de memoria» §5 ("La paginación modifica la fragmentación…"): a request of T
tokens on pages of B positions holds B·ceil(T/B) slots; its unused tail is
between 0 and B-1 positions.
«Paged Attention optimiza el uso de memoria» (paragraphs on the 16-token page table and on utilisation).
"""
from __future__ import annotations

from fractions import Fraction
from typing import Iterable

GIB = 1 << 30
GB = 10 ** 9


def kv_bytes_per_token(L: int, Hkv: int, d: int, b: int) -> int:
    """2·L·Hkv·d·b bytes of K and V per retained token («Servicio…presupuesto de memoria» §3)."""
    return 2 * L * Hkv * d * b


def kv_bytes(L: int, Hkv: int, d: int, b: int, lengths: Iterable[int]) -> int:
    """Bytes for all retained tokens: per-token cost times the sum of the
    stored positions of every sequence («¿Cuánta memoria reservar para la caché KV?», unequal lengths)."""
    return kv_bytes_per_token(L, Hkv, d, b) * sum(int(t) for t in lengths)


def blocks_for(T: int, B: int) -> int:
    """Pages a request of T tokens holds: T/B rounded up («Servicio…presupuesto de memoria» §5)."""
    if T < 0 or B < 1:
        raise ValueError("T >= 0 and B >= 1 required")
    return -(-T // B)


def allocated_slots(T: int, B: int) -> int:
    """Allocated capacity B·ceil(T/B) («Servicio…presupuesto de memoria» §5)."""
    return B * blocks_for(T, B)


def tail_waste(T: int, B: int) -> int:
    """Unused positions of the last page («Servicio…presupuesto de memoria» §5)."""
    return allocated_slots(T, B) - T


def mean_tail_waste(B: int, T_max: int) -> Fraction:
    """Exact mean tail waste for T uniform on 1..T_max («Servicio…presupuesto de memoria» §5)."""
    total = sum(tail_waste(T, B) for T in range(1, T_max + 1))
    return Fraction(total, T_max)


def mean_reservation_waste(reserve: int, T_max: int) -> Fraction:
    """Exact mean waste of reserving ``reserve`` slots per request for T
    uniform on 1..T_max (the contiguous scheme of «Servicio…presupuesto de memoria» §5)."""
    total = sum(reserve - T for T in range(1, T_max + 1))
    return Fraction(total, T_max)


def naive_utilisation(mean_len: float, max_len: int) -> float:
    """Fraction of a max-length contiguous reservation that holds tokens
    («Paged Attention optimiza el uso de memoria»: mean over maximum length)."""
    return mean_len / max_len


def paged_utilisation(lengths: Iterable[int], B: int) -> float:
    """Stored tokens over allocated page slots."""
    lengths = [int(t) for t in lengths]
    return sum(lengths) / sum(allocated_slots(T, B) for T in lengths)


def decode_kv_bytes(lengths: Iterable[int], Hkv: int, d: int, b: int, layers: int = 1) -> int:
    """K+V bytes one decode step reads to attend over ``lengths`` tokens in
    each of ``layers`` layers (the per-token cost over the attended tokens)."""
    return kv_bytes(layers, Hkv, d, b, lengths)
