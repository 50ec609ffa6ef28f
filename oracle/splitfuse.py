"""Dynamic SplitFuse token-budget composer (oracle side; test infrastructure).

What a forward pass holds ("DeepSpeed-FastGen 深度解析" §3.1-§3.2;
"第 15 章：推理引擎与部署", chunked prefill and its two worked scenarios):

* every running decode sequence contributes one token; the prompt tokens of
  a pass are limited by the budget left after the decodes
  (total = Σ chunk tokens + number of decodes ≤ budget);
* Split: a prompt longer than what is left is cut, the rest waits for the
  next passes; a prompt generates only in the pass that takes its last
  chunk, and decodes from the next pass on;
* Fuse: several prompts are packed into one pass, in arrival order, until the
  budget is exactly used;
* chunk = min(prompt tokens remaining, budget left): a 10,000-token prompt
  alone under a budget of 8192 runs as 8192 then 1808; next to 256 decodes a
  prompt gets at most 8192 − 256 = 7936 tokens.

Readings where the pages are silent: decodes that do not fit the budget wait
(the first ones in the order they started decoding are taken); a pass lists
the prompt chunks first, in arrival order, then the decodes; a decode row's
context is its prompt length plus the decodes it has run, this one included.

Each pass is a list of (seq_id, query tokens, context length after the pass).
Parity: pinned by the two scenarios and by invariants over random arrivals.
"""
from __future__ import annotations


class Composer:
    def __init__(self, budget: int):
        if budget <= 0:
            raise ValueError("budget must be positive")
        self.budget = budget
        self.queue = []    # [seq_id, prompt_len, done], arrival order
        self.running = []  # [seq_id, context], order they started decoding

    def add_prompt(self, seq_id, prompt_len: int) -> None:
        if prompt_len <= 0:
            raise ValueError("empty prompt")
        if any(q[0] == seq_id for q in self.queue) or any(r[0] == seq_id for r in self.running):
            raise ValueError("sequence exists")
        self.queue.append([seq_id, prompt_len, 0])

    def finish(self, seq_id) -> None:
        for lst in (self.running, self.queue):
            for i, e in enumerate(lst):
                if e[0] == seq_id:
                    del lst[i]
                    return
        raise KeyError("unknown sequence")

    def step(self):
        nd = min(len(self.running), self.budget)
        left = self.budget - nd
        chunks, done = [], []
        for q in self.queue:
            if left == 0:
                break
            c = min(q[1] - q[2], left)
            q[2] += c
            left -= c
            chunks.append((q[0], c, q[2]))
            if q[2] == q[1]:
                done.append(q)
        decodes = []
        for r in self.running[:nd]:
            r[1] += 1
            decodes.append((r[0], 1, r[1]))
        for q in done:
            self.queue.remove(q)
            self.running.append([q[0], q[1]])
        return chunks + decodes
