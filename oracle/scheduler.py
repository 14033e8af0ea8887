"""Oracle of the continuous-batching step scheduler.

TEST INFRASTRUCTURE ONLY (tests and the benchmark's checks import it; the
library never does). Plain Python over the oracle's own allocator model
(``oracle.Allocator``), written from the pages' description of one decode
step:

* "vLLM核心概念" §3.3 (the scheduler's loop, every decode step): go through
  the running requests; one that produced its end-of-sequence token or hit
  its token limit is done and its KV blocks are freed; the others stay; then
  new requests join from the waiting queue while free blocks remain; then one
  forward pass makes a token for every active request. §3.4: a waiting queue
  and a running batch, admission decided from the number of free blocks.
* "无 vLLM 环境下的 Paged-KV 与连续批处理调度" §3.1: admission checks the free
  page blocks; EOS (event kind 2) or the length limit (kind 3) end a request
  and its blocks are reclaimed at once.
* "连续批处理与KV缓存" §4.2: appending a block to a request returns "wait" when
  the free queue is empty; §4.4: on running out of memory, new requests are
  paused until blocks come back.

Readings where the pages are silent (the same ones the library documents):
the waiting queue is first come, first served and admission stops at the
first request that does not fit; admission needs the prompt's new blocks
plus `reserve` more; a request that waits is left out of the step; when
every running request waits, the most recently admitted one is preempted
(its blocks freed, put back at the queue front with its tokens so far as its
prompt), since otherwise no block would ever come back.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass

import numpy as np

from . import oracle as orc

ADMIT, EOS, MAX_LENGTH, PREEMPT, WAIT = 1, 2, 3, 4, 5


@dataclass
class _Req:
    rid: int
    prompt: int          # tokens written at admission
    max_new: int         # tokens it may still decode
    prefix: int          # oracle sequence holding a shared prompt prefix, or -1
    prefix_len: int
    length: int = 0      # tokens it holds while running
    made: int = 0        # tokens decoded since admission


class Scheduler:
    def __init__(self, alloc: orc.Allocator, max_batch: int, max_model_len: int, reserve: int = 1):
        self.a = alloc
        self.bs = alloc.block_size
        self.max_batch, self.max_model_len, self.reserve = max_batch, max_model_len, reserve
        self.max_blocks = -(-max_model_len // self.bs)
        self.queue: deque[_Req] = deque()
        self.running: list[_Req] = []
        self.paused = False
        self.last_batch: set[int] = set()
        self.totals = dict(admitted=0, finished_eos=0, finished_max_length=0, preempted=0, generated=0)

    def submit(self, rid: int, prompt: int, max_new: int, prefix: int = -1, prefix_len: int = 0):
        assert 1 <= prompt < self.max_model_len and max_new >= 1
        assert -(-min(prompt + max_new, self.max_model_len) // self.bs) <= self.a.num_blocks
        self.queue.append(_Req(rid, prompt, max_new, prefix, prefix_len if prefix >= 0 else 0))

    def _new_blocks(self, r: _Req) -> int:
        # logical blocks of the prompt, minus the full blocks it shares
        need = -(-r.prompt // self.bs)
        if r.prefix >= 0:
            if r.prompt == r.prefix_len:
                return 0
            need -= r.prefix_len // self.bs
        return need

    def step(self, eos=()):
        eos = set(int(x) for x in eos)
        assert eos <= self.last_batch
        events, pre_seqs, pre_first, pre_tokens, pre_slots = [], [], [], [], []

        # the running requests that are done give their blocks back
        still = []
        for r in self.running:
            if r.rid in eos:
                kind = EOS
            elif r.made >= r.max_new or r.length >= self.max_model_len:
                kind = MAX_LENGTH
            else:
                still.append(r)
                continue
            assert self.a.free(r.rid) == orc.OK
            events.append((r.rid, kind))
            self.totals["finished_eos" if kind == EOS else "finished_max_length"] += 1
            self.paused = False
        self.running = still

        # new requests join, in arrival order, while blocks remain
        while not self.paused and self.queue and len(self.running) < self.max_batch:
            r = self.queue[0]
            if self._new_blocks(r) + self.reserve > self.a.stats()["free"]:
                break
            self.queue.popleft()
            if r.prefix >= 0:
                assert self.a.fork(r.prefix, r.rid) == orc.OK
                n = r.prompt - r.prefix_len
                slots = np.zeros(0, dtype=np.int64)
                if n > 0:
                    st, slots = self.a.append([r.rid], [n])
                    assert st == orc.OK
                first = r.prefix_len
            else:
                st, slots = self.a.allocate(r.rid, r.prompt)
                assert st == orc.OK
                first = 0
            r.length, r.made = r.prompt, 0
            self.running.append(r)
            pre_seqs.append(r.rid)
            pre_first.append(first)
            pre_tokens.append(r.prompt - first)
            pre_slots.extend(int(x) for x in slots)
            events.append((r.rid, ADMIT))
            self.totals["admitted"] += 1

        # every active request takes its next position, or waits for a block
        while True:
            batch, slots, waiting = [], [], []
            for r in self.running:
                st, sl = self.a.append([r.rid], [1])
                if st == orc.OK:
                    batch.append(r.rid)
                    slots.append(int(sl[0]))
                else:
                    assert st == orc.NO_FREE_BLOCK
                    waiting.append(r.rid)
            if batch or not self.running:
                break
            r = self.running.pop()  # nobody can move: the youngest gives way
            assert self.a.free(r.rid) == orc.OK
            events.append((r.rid, PREEMPT))
            self.totals["preempted"] += 1
            self.queue.appendleft(_Req(r.rid, r.length, r.max_new - r.made, r.prefix, r.prefix_len))
        events.extend((rid, WAIT) for rid in waiting)
        if waiting:
            self.paused = True

        if batch:
            st, table, lens = self.a.table(batch, self.max_blocks)
            assert st == orc.OK
        else:
            table = np.zeros((0, self.max_blocks), dtype=np.int32)
            lens = np.zeros(0, dtype=np.int32)
        for r in self.running:
            if r.rid in batch:
                r.length += 1
                r.made += 1
                self.totals["generated"] += 1
        self.last_batch = set(batch)
        return {
            "seqs": np.array(batch, dtype=np.int64),
            "slots": np.array(slots, dtype=np.int64),
            "block_tables": table,
            "context_lens": lens,
            "max_blocks": self.max_blocks,
            "max_context_len": int(lens.max()) if len(lens) else 0,
            "prefill_seqs": np.array(pre_seqs, dtype=np.int64),
            "prefill_first": np.array(pre_first, dtype=np.int32),
            "prefill_tokens": np.array(pre_tokens, dtype=np.int32),
            "prefill_slots": np.array(pre_slots, dtype=np.int64),
            "events": events,
        }

    def stats(self) -> dict:
        s = self.a.stats()
        return dict(waiting=len(self.queue), running=len(self.running), **self.totals,
                    used_blocks=s["used"], total_blocks=self.a.num_blocks, paused=int(self.paused))
