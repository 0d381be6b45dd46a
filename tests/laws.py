"""Output laws of the verify step, shared by the GPU statistics tests and their CPU dry run.

A Case holds K+1 fixed target rows (and K draft rows) replicated over N independent rounds, each
with its own proposals and uniforms.  check_laws compares emitted tokens and accept lengths with
the closed forms of "Decodificação especulativa explicada" (gsantana.dev), sections "A regra de
amostragem por rejeição" and "Quanto mais rápido: a matemática": slot i, given that the round
reached it, is distributed as p_i; P(A >= a) = prod_{i<a} alpha_i, with alpha_i = sum min(p_i, q_i)
for a model drafter, sum r_i(x) p_i(x) for a one-hot drafter proposing x ~ r_i, and sum p_i q_i
for the sample-and-match mode.  Pearson chi-square with cells of expected count < 5 pooled; every
p-value must lie above 1e-3 divided by the number of tests in the case.
"""
import math

import numpy as np
import scipy.special
import scipy.stats
import torch

from oracle import closed_forms as cf
from speculative_decoding_verification_specdec_amd.inputs import (VerifyInputs, bf16_bits_to_f32,
                                                                  f32_to_bf16_bits)


def chi2_pooled(obs, exp):
    obs = np.asarray(obs, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    big = exp >= 5
    o, e = list(obs[big]), list(exp[big])
    if (~big).any() and exp[~big].sum() > 0:
        o.append(obs[~big].sum())
        e.append(exp[~big].sum())
    o, e = np.array(o), np.array(e)
    return float(scipy.stats.chi2.sf(((o - e) ** 2 / e).sum(), len(o) - 1))


class Case:
    """K+1 fixed target rows (and K draft rows) shared by N rounds; tensors on ``device``."""

    def __init__(self, V, K, N, seed, dtype="f32", T=1.0, z_sigma=2.0, draft_sigma=1.0,
                 onehot=False, ragged=False, device="cuda:0"):
        g = np.random.default_rng(seed)
        self.device = device
        z32 = (g.standard_normal((K + 1, V)) * z_sigma).astype(np.float32)
        if dtype == "bf16":
            bits = f32_to_bf16_bits(z32)
            z64 = bf16_bits_to_f32(bits).astype(np.float64)
            self.z_dev = torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            z64 = z32.astype(np.float64)
            self.z_dev = torch.from_numpy(z32).to(device)
        self.p = [scipy.special.softmax(z64[i] / T) for i in range(K + 1)]
        self.V, self.K, self.N, self.T = V, K, N, T
        self.onehot = onehot
        if onehot:
            # n-gram-like proposals: the target's argmax half the time, else a uniform id.
            self.r = [0.5 * np.eye(V)[int(np.argmax(self.p[i]))] + 0.5 / V for i in range(K)]
            self.q_dev = None
        else:
            dl = z64[:K] + g.standard_normal((K, V)) * draft_sigma
            q32 = scipy.special.softmax(dl, axis=1).astype(np.float32)
            self.q = q32.astype(np.float64)
            self.r = [self.q[i] / self.q[i].sum() for i in range(K)]
            self.q_dev = torch.from_numpy(q32).to(device)
        self.x = np.stack([g.choice(V, size=N, p=self.r[i]) for i in range(K)], 1).astype(np.int32)
        self.u = g.random((N, K + 1), dtype=np.float32)
        self.kb = g.integers(0, K + 1, size=N).astype(np.int32) if ragged else None

    def run(self, match=False):
        """The HIP path through the C ABI: (accept_len, out_tokens) as numpy."""
        from speculative_decoding_verification_specdec_amd import (specdec_verify,
                                                                   specdec_verify_match)
        N, dev = self.N, self.device
        logits = self.z_dev.unsqueeze(0).expand(N, -1, -1).contiguous()
        draft = (None if self.q_dev is None
                 else self.q_dev.unsqueeze(0).expand(N, -1, -1).contiguous())
        x = torch.from_numpy(self.x).to(dev)
        T = torch.full((N,), self.T, dtype=torch.float32, device=dev)
        u = torch.from_numpy(self.u).to(dev)
        nd = None if self.kb is None else torch.from_numpy(self.kb).to(dev)
        if match:
            acc, tok, _ = specdec_verify_match(logits, x, T, u, num_draft=nd)
        else:
            oh = torch.ones(N, dtype=torch.uint8, device=dev) if self.onehot else None
            acc, tok, _ = specdec_verify(logits, draft, x, T, u, draft_onehot=oh, num_draft=nd)
        torch.cuda.synchronize()
        del logits, draft
        return acc.cpu().numpy(), tok.cpu().numpy()

    def host_inputs(self):
        """The same rounds as a host VerifyInputs batch (for the oracle)."""
        N, K, V = self.N, self.K, self.V
        z = self.z_dev.cpu()
        if z.dtype == torch.bfloat16:
            bits, dt = z.view(torch.int16).numpy().view(np.uint16), "bf16"
        else:
            bits, dt = z.numpy(), "f32"
        logits = np.ascontiguousarray(np.broadcast_to(bits, (N, K + 1, V)))
        draft = (None if self.q_dev is None else
                 np.ascontiguousarray(np.broadcast_to(self.q_dev.cpu().numpy(), (N, K, V))))
        oh = np.ones(N, np.uint8) if self.onehot else None
        return VerifyInputs(logits, dt, draft, oh, self.x, self.kb,
                            np.full(N, self.T, np.float32), self.u, name="law_case")

    def alphas(self, match=False):
        if match:
            return [float(np.dot(self.p[i], self.q[i])) for i in range(self.K)]
        if self.onehot:
            return [float(np.dot(self.r[i], self.p[i])) for i in range(self.K)]
        return [cf.acceptance_rate(self.p[i], self.q[i]) for i in range(self.K)]


def check_laws(case, acc, tok, alphas):
    K = case.K
    kb = np.full(case.N, K) if case.kb is None else case.kb
    assert ((acc >= 0) & (acc <= kb)).all()
    pvals = {}
    for i in range(K + 1):                       # slot i, given the round reached it
        sel = (acc >= i) & (kb >= i)
        if sel.sum() < 200:
            continue
        obs = np.bincount(tok[sel, i], minlength=case.V)
        assert obs.size == case.V, "token id out of range"
        pvals[f"slot{i}"] = chi2_pooled(obs, sel.sum() * case.p[i])
        # Slots past the emitted one stay empty.
        assert (tok[(acc < i) & (kb >= i), i] == -1).all()
    for k in np.unique(kb[kb > 0]):              # accept length of the rounds drafting k
        sel = kb == k
        law = cf.accept_length_law(alphas[:k])
        pvals[f"A|k={k}"] = chi2_pooled(np.bincount(acc[sel], minlength=k + 1), sel.sum() * law)
        mean, se = (acc[sel] + 1).mean(), (acc[sel] + 1).std() / math.sqrt(sel.sum())
        assert abs(mean - cf.expected_tokens_from_law(alphas[:k])) < 5 * se + 1e-12, (k, mean)
    print("[pvals]", {k: round(v, 4) for k, v in pvals.items()}, flush=True)
    assert min(pvals.values()) > 1e-3 / len(pvals), pvals
