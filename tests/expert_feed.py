"""Expert weights for the CPU oracle at the GLM shape, decoded ahead of use.

``oracle.forward`` asks for one routed expert at a time, in ascending expert
order, and decodes its bf16 weights to float64 before the products.  At the
GLM shape that decoding (three 2048 x 6144 matrices per expert) is most of the
oracle's time, so this feed runs the oracle's own ``decode`` on the next
experts in worker threads and hands over the float64 arrays, which ``decode``
then passes through unchanged in value.  Test infrastructure only; no
arithmetic of the layer happens here.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Iterable

import oracle


class ExpertFeed:
    def __init__(self, get: Callable[[int], tuple], order: Iterable[int], threads: int = 8,
                 ahead: int = 12):
        self.get = get
        self.order = [int(e) for e in order]
        self.ahead = ahead
        self.ex = ThreadPoolExecutor(threads)
        self.fut = {}
        self.pos = 0
        self._fill()

    def _fill(self):
        while self.pos < len(self.order) and len(self.fut) < self.ahead:
            e = self.order[self.pos]
            self.pos += 1
            self.fut[e] = self.ex.submit(lambda e=e: tuple(oracle.decode(a) for a in self.get(e)))

    def __call__(self, e: int):
        f = self.fut.pop(int(e), None)
        if f is None:
            return self.get(int(e))
        v = f.result()
        self._fill()
        return v

    def close(self):
        self.ex.shutdown(wait=True, cancel_futures=True)
        self.fut.clear()
