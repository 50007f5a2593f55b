"""CPU tests: the page-allocator oracle against its pins, and the pins against
planted mistakes in it."""
from collections import deque

import numpy as np
import pytest

import oracle.alloc_oracle as A
from tests import alloc_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_alloc_oracle_pin(pin):
    pin()


_orig_new_pages = A.new_pages


def _lifo_allocate(self, cached_len, device_len, page_size):
    need = sum(A.new_pages(c, d, page_size) for c, d in zip(cached_len, device_len))
    if need > len(self.rows):
        return None
    return [self.rows.pop() for _ in range(need)]


def _partial_allocate(self, cached_len, device_len, page_size):
    need = sum(A.new_pages(c, d, page_size) for c, d in zip(cached_len, device_len))
    need = min(need, len(self.rows))
    return [self.rows.popleft() for _ in range(need)]


def _free_front(self, rows):
    rows = [int(r) for r in rows]
    if len(self.rows) + len(rows) > self.capacity:
        return False
    self.rows.extendleft(reversed(rows))
    return True


MUTANTS = {
    "floor_pages": ("new_pages", lambda c, d, s: (int(d) // s - int(c) // s) if 0 <= int(c) <= int(d) else 0),
    "pages_for_bad_lengths": ("new_pages", lambda c, d, s: _orig_new_pages(min(c, d), max(c, d), s)),
    "pages_over_device_len_only": ("new_pages", lambda c, d, s: -(-int(d) // s) if 0 <= int(c) <= int(d) else 0),
    "lifo": ("FreeList.allocate", _lifo_allocate),
    "partial_on_shortage": ("FreeList.allocate", _partial_allocate),
    "free_to_front": ("FreeList.free", _free_front),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_alloc_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if attr.startswith("FreeList."):
        monkeypatch.setattr(A.FreeList, attr.split(".")[1], fn)
    else:
        monkeypatch.setattr(A, attr, fn)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
