"""Helpers for the GPU parity tests: run the same seeded steps through the
HIP library (via the Python binding) and through the CPU oracle, and compare.

Bars (stated once, used everywhere):
  * lengths, positions and slot indices: bit-exact;
  * float32 outputs: max abs error <= 1e-5;
  * bfloat16 outputs: max abs error <= 2e-2 and ||got - ref|| / ||ref|| <= 1e-2
    per (layer, step) tensor;
  * padded queries and idle rows: exactly 0.
"""

import sys

import numpy as np
import torch

import kv_cached_gqa_append_amd as K
import oracle
import workloads as wl

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().double().cpu().numpy()


def check_outputs(got, ref, n_new, dtype, what):
    """got, ref: (B, C, Hq, D) float64 arrays."""
    C = got.shape[1]
    pad = np.arange(C)[None, :] >= np.asarray(n_new)[:, None]
    assert np.all(got[pad] == 0.0), f"{what}: padded/idle outputs are not exactly zero"
    d = np.abs(got - ref)
    mx = float(d.max()) if d.size else 0.0
    if dtype == "f32":
        assert mx <= F32_MAX_ABS, f"{what}: max abs {mx:.3e} > {F32_MAX_ABS}"
        return mx, 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / nrm if nrm > 0 else 0.0
    assert mx <= BF16_MAX_ABS, f"{what}: max abs {mx:.3e} > {BF16_MAX_ABS}"
    assert rel <= BF16_REL_L2, f"{what}: rel l2 {rel:.3e} > {BF16_REL_L2}"
    return mx, rel


class Pair:
    """A GPU cache and an oracle driven by the same seeded inputs."""

    def __init__(self, work: wl.Workload, device="cuda", poison=False, tag=""):
        self.work = work
        self.tag = tag
        self.device = torch.device(device)
        cfg = K.config_from_workload(work)
        buf = None
        if poison:
            # 0xFF bytes are NaN in both bf16 and fp32: every row the path must
            # never read stays NaN.
            buf = torch.full((K.kvc_nbytes(cfg, K.KVC_NB_ALLOC),), 255, dtype=torch.uint8,
                             device=self.device)
        self.cache = K.Cache(cfg, self.device, buffer=buf)
        self.ref = oracle.OracleCache(work.batch, work.n_q_head, work.n_kv_head, work.head_dim,
                                      work.max_len, work.window, work.rope_base,
                                      joint=work.joint or None)
        self.step_no = 0
        self.worst = 0.0
        self.worst_rel = 0.0

    def step(self, n_new, C, check=True, check_slots=True, fused=False):
        """One step over every layer; ``fused`` drives it through
        kvc_append_attend instead of kvc_append + kvc_attend."""
        w = self.work
        n_new = np.asarray(n_new, dtype=np.int64)
        lens_before = self.ref.lens.copy()
        layers = [wl.step_qkv(w, l, self.step_no, C, self.tag) for l in range(w.n_layer)]
        outs, slots = [], []
        for l, (q, k, v) in enumerate(layers):
            so = torch.full((w.batch, C), -7, dtype=torch.int32, device=self.device)
            if fused:
                outs.append(self.cache.append_attend(l, q.to(self.device), k.to(self.device),
                                                     v.to(self.device), n_new, slot_out=so))
            else:
                self.cache.append(l, k.to(self.device), v.to(self.device), n_new, slot_out=so)
                outs.append(self.cache.attend(l, q.to(self.device)))
            slots.append(so)
        self.cache.advance()
        exp = self.ref.step(n_new, [tuple(f64(t) for t in x) for x in layers], compute=check)
        torch.cuda.synchronize()
        if check_slots:
            for l in range(w.n_layer):
                want = oracle.slot_indices(lens_before, n_new, C, w.window[l], w.max_len,
                                           w.use_ring)
                got = slots[l].cpu().numpy()
                assert np.array_equal(got, want), f"layer {l} step {self.step_no}: slots {got} != {want}"
        if check:
            for l in range(w.n_layer):
                mx, rel = check_outputs(f64(outs[l]), exp[l], n_new, w.dtype,
                                        f"{w.name} layer {l} step {self.step_no}")
                self.worst = max(self.worst, mx)
                self.worst_rel = max(self.worst_rel, rel)
        assert self.cache.lens() == [int(x) for x in self.ref.lens]
        assert self.cache.device_lens().tolist() == [int(x) for x in self.ref.lens]
        self.step_no += 1
        return outs

    def reset(self, rows):
        self.cache.reset(rows)
        self.ref.reset(rows)

    def set_first(self, rows, first):
        self.cache.set_first(rows, first)
        self.ref.set_first(rows, first)

    def admit(self, rows, src: "Pair", src_rows):
        self.cache.admit(rows, src.cache, src_rows)
        self.ref.admit(rows, src.ref, src_rows)

    def check_cache_rows(self, layer):
        """Stored K (rotated) and V of every live row against the oracle's raw
        history: V bit-exact; K is the rotation computed in float32 and
        rounded to the dtype, so it must lie between the roundings of
        R(k, pos) -/+ e, e = 2^-21 (|x_d| + |x_partner|) bounding the float32
        error of the table entries and the two products (float32 caches:
        within 1e-6)."""
        w = self.work
        kview = self.cache.k_view(layer).float().cpu().numpy()
        vview = self.cache.v_view(layer).float().cpu().numpy()
        W = w.window[layer]
        ring = oracle.cache.is_ring(W, w.max_len, w.use_ring)
        for b in range(w.batch):
            L = int(self.ref.lens[b])
            hk, hv = self.ref.history(layer, b)
            lo = max(0, L - W) if ring else 0
            pos = np.arange(lo, L)
            if pos.size == 0:
                continue
            slot = pos % W if ring else pos
            krot = oracle.rope.rotate(hk[lo:L], pos, w.rope_base)     # (n, Hkv, D) fp64
            got_k = kview[b][:, slot, :].transpose(1, 0, 2)           # (n, Hkv, D)
            got_v = vview[b][:, slot, :].transpose(1, 0, 2)
            assert np.array_equal(got_v, hv[lo:L]), f"layer {layer} row {b}: V differs"
            if w.dtype == "f32":
                assert np.abs(got_k - krot).max() <= 1e-6, f"layer {layer} row {b}: K"
            else:
                raw = np.abs(hk[lo:L])
                e = 2.0 ** -21 * (raw + np.roll(raw, w.head_dim // 2, axis=-1))
                lo_b = torch.from_numpy(krot - e).float().to(torch.bfloat16).float().numpy()
                hi_b = torch.from_numpy(krot + e).float().to(torch.bfloat16).float().numpy()
                bad = (got_k < lo_b) | (got_k > hi_b)
                assert not bad.any(), (f"layer {layer} row {b}: K is not the dtype rounding of "
                                       f"its rotation ({int(bad.sum())} elements)")


class SampledOracle:
    """The oracle on a few rows of a workload too large to check in full.

    It keeps the raw history of the sampled rows only.  Tokens appended on
    the GPU are recorded as they go and handed to the oracle in one step when
    a check needs them (the oracle is chunk-invariant: pinned by the
    chunked-equals-single check).  ``check`` compares chosen queries of the
    current step against ``OracleCache.query_rows``.
    """

    def __init__(self, work, rows):
        self.work = work
        self.rows = [int(r) for r in rows]
        self.ref = oracle.OracleCache(len(self.rows), work.n_q_head, work.n_kv_head,
                                      work.head_dim, work.max_len, work.window, work.rope_base)
        self.pending = [[[] for _ in self.rows] for _ in range(work.n_layer)]

    def record(self, layer, k, v, n_new):
        """Remember the valid tokens of the sampled rows (k, v on the GPU)."""
        for j, b in enumerate(self.rows):
            n = int(n_new[b])
            if n:
                self.pending[layer][j].append((f64(k[b, :n]), f64(v[b, :n])))

    def catch_up(self):
        """Append every recorded token to the oracle in one step."""
        w = self.work
        counts = [sum(x[0].shape[0] for x in self.pending[0][j]) for j in range(len(self.rows))]
        for l in range(w.n_layer):
            assert [sum(x[0].shape[0] for x in self.pending[l][j])
                    for j in range(len(self.rows))] == counts
        C = max(counts)
        if C == 0:
            return
        layers = []
        for l in range(w.n_layer):
            hk = w.n_kv_head[l]
            K = np.zeros((len(self.rows), C, hk, w.head_dim))
            V = np.zeros_like(K)
            for j in range(len(self.rows)):
                if counts[j]:
                    K[j, :counts[j]] = np.concatenate([x[0] for x in self.pending[l][j]])
                    V[j, :counts[j]] = np.concatenate([x[1] for x in self.pending[l][j]])
            q = np.broadcast_to(np.float64(0.0), (len(self.rows), C, w.n_q_head, w.head_dim))
            layers.append((q, K, V))
        self.ref.step(np.asarray(counts), layers, compute=False)
        self.pending = [[[] for _ in self.rows] for _ in range(w.n_layer)]

    def check_step(self, n_new, qkv, outs, queries, what):
        """The current step on the sampled rows: append its tokens to the
        oracle, compare outputs of ``queries(b, n) -> indices`` for every
        sampled row and layer, then advance.  qkv[l] = (q, k, v) on the GPU;
        outs[l] the GPU outputs.  Returns (max abs, max rel l2)."""
        w = self.work
        self.catch_up()
        nn = np.array([int(n_new[b]) for b in self.rows])
        worst, worst_rel = 0.0, 0.0
        for l in range(w.n_layer):
            q, k, v = qkv[l]
            C = q.shape[1]
            sel = torch.tensor(self.rows, device=q.device)
            ks, vs = f64(k[sel]), f64(v[sel])
            qz = np.broadcast_to(np.float64(0.0), (len(self.rows), C, w.n_q_head, w.head_dim))
            self.ref.layer_step(l, nn, qz, ks, vs, compute=False)
            got_all = f64(outs[l][sel])
            for j, b in enumerate(self.rows):
                n = int(nn[j])
                if n == 0:
                    assert np.all(got_all[j] == 0.0), f"{what}: idle row {b} layer {l} not zero"
                    continue
                idx = np.asarray(queries(b, n), dtype=np.int64)
                exp = self.ref.query_rows(l, j, n, f64(q[b, :n]), idx)
                got = got_all[j, idx]
                d = np.abs(got - exp)
                mx = float(d.max())
                rel = float(np.linalg.norm(got - exp) / max(np.linalg.norm(exp), 1e-300))
                assert mx <= BF16_MAX_ABS, f"{what}: row {b} layer {l} max abs {mx:.3e}"
                assert rel <= BF16_REL_L2, f"{what}: row {b} layer {l} rel l2 {rel:.3e}"
                assert np.all(got_all[j, n:] == 0.0), f"{what}: row {b} padded outputs not zero"
                worst, worst_rel = max(worst, mx), max(worst_rel, rel)
        self.ref.advance(nn)
        return worst, worst_rel
