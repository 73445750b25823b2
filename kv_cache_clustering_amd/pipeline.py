"""Algorithm 1 runtime: a clustered K/V cache driven through prefill rounds and decode steps.

Chelsea review, section 三, Algorithm 1: after prefill, cluster while s >= B + g (budget
B = R * (n + Gamma)); each decode step appends k, v with degree 1, attends with
O = Softmax(q K^T / sqrt(d) + log N) V, and clusters when s >= B + g.  CentroidKV page,
渐进式调度: r is annealed over rounds.

Every length is known on the host in closed form (schedule.Algorithm1), so driving the
device needs no read-back: the whole loop is a sequence of asynchronous library calls on
the current stream.  With the device-side trigger (csm_compress_triggered) the round of a
step is decided on the device from each slice's length and round counter, so many steps can
also be captured in one HIP graph (capture_loop / run_loop).  All sequences of a batch share one
prefill length and therefore one schedule; slices flagged outlier are never clustered and keep
growing.
"""

import torch

from . import _lib as lib
from .schedule import Algorithm1


class ClusteredKVCache:
    """K, V: [S, cap, d] (S = batch * layers * H_kv); N: [S, cap] int32; lens: [S] int32.

    The tensors are used in place.  `n` is the common prefill length of every slice.
    """

    def __init__(self, K, V, N, lens, *, H_q, H_kv, n, R, Gamma, g=32, n1=16, n2=64, c=256,
                 r_init=0.5, delta=0.05, r_min=0.1, outlier_mask=None, observer=None):
        """observer: optional object with before_round(cache, r) and
        after_round(cache, r, best_b, selected, src_pos); rounds then record their decisions
        (csm_compress_debug, same kernel)."""
        self.K, self.V, self.N, self.lens = K, V, N, lens
        self.observer = observer
        self.H_q, self.H_kv = H_q, H_kv
        self.n1, self.n2, self.c = n1, n2, c
        self.mask = outlier_mask
        self.has_outliers = outlier_mask is not None and bool(outlier_mask.any())
        self.sched = Algorithm1(n=n, R=R, Gamma=Gamma, g=g, n1=n1, n2=n2, c=c, r_init=r_init,
                                delta=delta, r_min=r_min)
        self.step_index = 0
        self.outlier_len = n
        dev = K.device
        cap = K.shape[1]
        self.ws_csm = lib.new_workspace(lib.csm_workspace_bytes(K, n1, n2, c, max_len=cap), dev)
        self.ws_dec = lib.new_workspace(lib.decode_workspace_bytes(K, H_q, H_kv, max_len=cap), dev)
        groups = K.shape[0] // H_kv
        self.out = torch.empty((groups, H_q, K.shape[2]), dtype=torch.float32, device=dev)

    @property
    def max_len(self):
        """Host-known bound on every slice length."""
        return max(self.sched.s, self.outlier_len if self.has_outliers else 0)

    def _round(self, r, s_before):
        """One clustering round in place; s_before (host-known length of the compressed slices
        before it) bounds the launch: outlier slices are not read, so they need no cover."""
        max_len = s_before
        if self.observer is None:
            lib.csm_compress(self.K, self.V, self.N, self.lens, self.n1, self.n2, self.c, r,
                             self.mask, max_len=max_len, workspace=self.ws_csm)
            return
        self.observer.before_round(self, r)
        taps = lib.csm_compress_debug(self.K, self.V, self.N, self.lens, self.n1, self.n2, self.c,
                                      r, self.mask, max_len=max_len, workspace=self.ws_csm)
        self.observer.after_round(self, r, *taps[:3])

    def prefill(self):
        """Cluster until the cache is under budget; returns the r of every round run."""
        rs = []
        while self.sched.over_budget():
            s_before = self.sched.s
            r = self.sched.next_round(0)
            self._round(r, s_before)
            rs.append(r)
        return rs

    def decode_step(self, q, k_new, v_new, out=None):
        """Append, attend, then cluster if the trigger fires.  Returns (O, r or None)."""
        self.step_index += 1
        self.sched.append()
        self.outlier_len += 1
        O, _ = lib.kv_append_decode_attn_logn(q, self.K, self.V, self.N, self.lens, self.H_q,
                                              self.H_kv, k_new, v_new,
                                              out=self.out if out is None else out,
                                              max_len=self.max_len, workspace=self.ws_dec)
        r = None
        if self.sched.over_budget():
            s_before = self.sched.s
            r = self.sched.next_round(self.step_index)
            self._round(r, s_before)
        return O, r

    def capture_decode(self):
        """Capture one decode step (append + attention, one fused call) into a HIP graph.

        The launch bounds are fixed at the cache capacity (the kernels read the actual
        lengths on the device), so one graph serves every step.  Step inputs are read from
        the static buffers q_in, k_in, v_in; the output lands in self.out.  Clustering
        rounds stay outside the graph (they are rare and their r changes).
        """
        S, cap, d = self.K.shape
        dev = self.K.device
        groups = S // self.H_kv
        self.q_in = torch.zeros((groups, self.H_q, d), dtype=self.K.dtype, device=dev)
        self.k_in = torch.zeros((S, d), dtype=self.K.dtype, device=dev)
        self.v_in = torch.zeros((S, d), dtype=self.K.dtype, device=dev)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            lib.kv_append_decode_attn_logn(self.q_in, self.K, self.V, self.N, self.lens, self.H_q,
                                           self.H_kv, self.k_in, self.v_in, out=self.out,
                                           max_len=cap, workspace=self.ws_dec)
        self.graph = graph

    def decode_step_graph(self, q=None, k_new=None, v_new=None):
        """decode_step through the captured graph.  Inputs, when given, are copied into the
        static buffers first.  Returns (O, r or None)."""
        if q is not None:
            self.q_in.copy_(q)
            self.k_in.copy_(k_new)
            self.v_in.copy_(v_new)
        self.step_index += 1
        self.graph.replay()
        self.sched.append()
        self.outlier_len += 1
        r = None
        if self.sched.over_budget():
            s_before = self.sched.s
            r = self.sched.next_round(self.step_index)
            self._round(r, s_before)
        return self.out, r

    # ------------------------------------------------------------ device-side trigger
    def _device_schedule(self):
        """Per-slice trigger threshold ceil(B + g) and round counter (the device's copy of the
        schedule state), created on first use from the host bookkeeping."""
        if getattr(self, "thr", None) is None:
            import math
            S = self.K.shape[0]
            dev = self.K.device
            if self.sched.budget is None:
                raise ValueError("the device trigger needs a budget (R)")
            t = math.ceil(self.sched.budget + self.sched.g)
            self.thr = torch.full((S,), t, dtype=torch.int32, device=dev)
            self.round_idx = torch.full((S,), self.sched.j, dtype=torch.int32, device=dev)
        return self.thr, self.round_idx

    def _triggered_round(self, max_len, observe=True):
        """One csm_compress_triggered call: every slice at its threshold runs a round with its
        own annealed r.  An observer with before_device_round(cache) / after_device_round(cache)
        sees the cache around the call (not while a graph is being captured)."""
        thr, idx = self._device_schedule()
        obs = self.observer if observe and hasattr(self.observer, "before_device_round") else None
        if obs is not None:
            obs.before_device_round(self)
        lib.csm_compress_triggered(self.K, self.V, self.N, self.lens, thr, idx, self.n1, self.n2,
                                   self.c, self.sched.r_init, self.sched.delta, self.sched.r_min,
                                   self.mask, max_len=max_len, workspace=self.ws_csm)
        if obs is not None:
            obs.after_device_round(self)

    def prefill_device(self):
        """prefill with the trigger and r decided on the device: one triggered call for each
        round the host bookkeeping predicts (each slice runs when its length is at the threshold,
        with r from its own round counter).  Returns the r the host expects of each round."""
        self._device_schedule()  # the device's round counters start at the rounds run so far
        rs = []
        while self.sched.over_budget():
            s_before = self.sched.s
            rs.append(self.sched.next_round(0))
            self._triggered_round(s_before)
        return rs

    def _host_step(self):
        """Advance the host bookkeeping by one decode step (append, then the trigger)."""
        self.step_index += 1
        self.sched.append()
        self.outlier_len += 1
        if self.sched.over_budget():
            return self.sched.next_round(self.step_index)
        return None

    def decode_step_device(self, q, k_new, v_new, out=None):
        """decode_step with the trigger and r decided on the device: nothing on the host
        decides whether the round runs.  The host bookkeeping is advanced in closed form so
        that it keeps the same lengths.  Returns (O, r the host expects, or None)."""
        self.step_index += 1
        self.sched.append()
        self.outlier_len += 1
        bound = self.max_len  # lengths after the append, before any round
        O, _ = lib.kv_append_decode_attn_logn(q, self.K, self.V, self.N, self.lens, self.H_q,
                                              self.H_kv, k_new, v_new,
                                              out=self.out if out is None else out,
                                              max_len=bound, workspace=self.ws_dec)
        self._triggered_round(self.sched.s)  # slices that can run share this length
        r = self.sched.next_round(self.step_index) if self.sched.over_budget() else None
        return O, r

    def capture_loop(self, steps):
        """Capture `steps` decode steps (append, attention, device-triggered round) in one HIP
        graph.  Inputs are read from the static buffers loop_q [steps, groups, H_q, d],
        loop_k / loop_v [steps, S, d]; outputs land in loop_out [steps, groups, H_q, d].
        Launch bounds: attention over the capacity, rounds over the trigger threshold plus
        the steps of one replay (a round runs as soon as a slice reaches the threshold)."""
        S, cap, d = self.K.shape
        dev = self.K.device
        groups = S // self.H_kv
        thr, _ = self._device_schedule()
        round_bound = min(cap, max(int(thr.max().item()), self.sched.s) + steps)
        if self.ws_csm.numel() < lib.csm_workspace_bytes(self.K, self.n1, self.n2, self.c,
                                                         max_len=round_bound):
            raise ValueError("CSM workspace too small for the loop's launch bound")
        self.loop_q = torch.zeros((steps, groups, self.H_q, d), dtype=self.K.dtype, device=dev)
        self.loop_k = torch.zeros((steps, S, d), dtype=self.K.dtype, device=dev)
        self.loop_v = torch.zeros((steps, S, d), dtype=self.K.dtype, device=dev)
        self.loop_out = torch.empty((steps, groups, self.H_q, d), dtype=torch.float32, device=dev)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                lib.kv_append_decode_attn_logn(self.loop_q[i], self.K, self.V, self.N, self.lens,
                                               self.H_q, self.H_kv, self.loop_k[i],
                                               self.loop_v[i], out=self.loop_out[i], max_len=cap,
                                               workspace=self.ws_dec)
                self._triggered_round(round_bound, observe=False)
        self.loop_graph = graph
        self.loop_steps = steps

    def run_loop(self, q=None, k_new=None, v_new=None):
        """Replay the captured loop once (inputs, when given, are copied into the static
        buffers first).  Returns (loop_out, the r of every round the host bookkeeping expects
        as (step, r) pairs)."""
        if q is not None:
            self.loop_q.copy_(q)
            self.loop_k.copy_(k_new)
            self.loop_v.copy_(v_new)
        self.loop_graph.replay()
        rounds = []
        for _ in range(self.loop_steps):
            r = self._host_step()
            if r is not None:
                rounds.append((self.step_index, r))
        return self.loop_out, rounds

    def check_errors(self):
        """Synchronise and raise if a kernel flagged a bad length since the cache was built
        (the error words are sticky)."""
        for word in (self.ws_csm, self.ws_dec):
            rc = lib.read_error(word)
            if rc != lib.OK:
                raise lib.CsmkvError(rc, "device")
