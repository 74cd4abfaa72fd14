"""Every entry point replayed from a captured HIP graph (torch.cuda.CUDAGraph).

The library allocates nothing, never synchronizes and clears no memory with
memset, so a whole chain can be captured once and replayed.  Each test runs
the chain eagerly, captures it, then replays it several times with its
outputs poisoned and unrelated eager work in between, and requires every
replay to reproduce the eager result bit for bit (all kernels add in a fixed
order, so the results are deterministic).
"""
import numpy as np
import pytest
import torch

import synth
from input_adaptive_reduced_rmm_amd import binding as R
from _parity import dev_tensor

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def _replay_matches(chain, outputs, reps=4):
    chain()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for rep in range(reps):
        for o in outputs:
            if o.dtype in (torch.int32, torch.int8):
                o.fill_(-7)
            else:
                o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager run"
        _ = (torch.arange(1000, device=DEV, dtype=torch.float32) * rep).sum().item()   # unrelated eager work
    del g


def test_graph_projection_chain_packed_path():
    """m >= 1024: column norms, top-k, A pack, B pack and the persistent GEMM."""
    m, d, n, rho = 2048, 1536, 1280, 0.55
    A = dev_tensor(synth.outlier_activations(synth.stream(1, 91, 1), m, d, 0.01, 20.0), BF)
    B = dev_tensor(synth.weight(synth.stream(1, 91, 2), d, n), BF)
    k = R.rmm_k_from_rho(rho, d)
    sc = torch.empty(d, dtype=torch.float32, device=DEV)
    idx = torch.empty(R.rmm_k_pad(k), dtype=torch.int32, device=DEV)
    Y = torch.empty((m, n), dtype=BF, device=DEV)
    ws_c = torch.empty(max(R.rmm_colnorm_workspace_bytes(BF, m, d, 1), 256), dtype=torch.uint8, device=DEV)
    ws_g = torch.empty(max(R.rmm_gemm_workspace_bytes(BF, m, n, k), 256), dtype=torch.uint8, device=DEV)

    def chain():
        R.rmm_colnorm(A, out=sc, ws=ws_c)
        R.rmm_topk(sc, k, out=idx)
        R.rmm_gemm(A, B, idx, k, out=Y, ws=ws_g)

    _replay_matches(chain, [sc, idx, Y])


def test_graph_qk_pv_chain():
    L, Hq, Hkv, kf, kt = 600, 4, 2, 64, 300
    Q, Kt, V = synth.attention_qkv(3, 91, L, Hq, Hkv, 128)
    Qd, Ktd, Vd = dev_tensor(Q, BF), dev_tensor(Kt, BF), dev_tensor(V, BF)
    P = synth.causal_probs(Q, Kt, 128 ** -0.5).to(DEV)
    S = torch.empty((Hq, L, L), dtype=torch.float32, device=DEV)
    O = torch.empty((L, Hq, 128), dtype=BF, device=DEV)
    iq = torch.empty((Hq, R.rmm_k_pad(kf)), dtype=torch.int32, device=DEV)
    ip = torch.empty((Hq, R.rmm_k_pad(kt)), dtype=torch.int32, device=DEV)
    wq = torch.empty(R.rmm_qk_workspace_bytes(L, Hq, 128, kf), dtype=torch.uint8, device=DEV)
    wp = torch.empty(R.rmm_pv_workspace_bytes(Hq, L, L, kt), dtype=torch.uint8, device=DEV)

    def chain():
        R.rmm_qk(Qd, Ktd, kf, S=S, idx=iq, ws=wq, causal=True)
        R.rmm_pv(P, Vd, kt, O=O, idx=ip, ws=wp, causal=True)

    # the causal QK^T leaves tiles above the diagonal unwritten: compare the lower triangle via a mask
    lower = torch.ones((L, L), dtype=torch.bool, device=DEV).tril_()
    S.zero_()

    def chain_masked():
        chain()
        S.masked_fill_(~lower, 0.0)

    _replay_matches(chain_masked, [S, O, iq, ip])


@pytest.mark.parametrize("Lq,Lk", [(500, 500), (1, 2000), (9, 700)])
def test_graph_fused_attention(Lq, Lk):
    """Prefill passes and the few-token decode passes, with the column scores of O."""
    Hq, Hkv, kf, kt = 4, 2, 64, Lk // 2
    Q, Kt, V = synth.attention_operands(synth.WORKLOADS["attn-32h-4k"], L=Lk, Hq=Hq, Hkv=Hkv)
    Qd = dev_tensor(np.ascontiguousarray(Q[Lk - Lq:]), BF)
    Ktd, Vd = dev_tensor(Kt, BF), dev_tensor(V, BF)
    O = torch.empty((Lq, Hq, 128), dtype=BF, device=DEV)
    If = torch.empty((Hq, R.rmm_k_pad(kf)), dtype=torch.int32, device=DEV)
    It = torch.empty((Hq, R.rmm_k_pad(kt)), dtype=torch.int32, device=DEV)
    ts = torch.empty((Hq, Lk), dtype=torch.float32, device=DEV)
    os_ = torch.empty((Hq, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty(R.rmm_attention_workspace_bytes(Lq, Lk, Hq, 128, kf, kt), dtype=torch.uint8, device=DEV)

    def chain():
        R.rmm_attention(Qd, Ktd, Vd, kf, kt, O=O, idx_feat=If, idx_tok=It, tok_scores=ts, ws=ws, causal=True,
                        o_scores=os_)

    _replay_matches(chain, [O, If, It, ts, os_])


def test_graph_w8_and_producers():
    """INT8-weight product on the many-row path (dequantized kept rows) and both producers."""
    m, d, n, k = 300, 1024, 512, 700
    A = dev_tensor(synth.outlier_activations(synth.stream(4, 91, 1), m, d, 0.01, 20.0), BF)
    q, sc = synth.int8_per_column(synth.weight(synth.stream(4, 91, 2), d, n))
    qd, scd = dev_tensor(q, torch.int8), dev_tensor(sc, torch.float32)
    s = torch.empty(d, dtype=torch.float32, device=DEV)
    idx = torch.empty(R.rmm_k_pad(k), dtype=torch.int32, device=DEV)
    Y = torch.empty((m, n), dtype=BF, device=DEV)
    ws_c = torch.empty(max(R.rmm_colnorm_workspace_bytes(BF, m, d, 1), 256), dtype=torch.uint8, device=DEV)
    ws_w = torch.empty(max(R.rmm_gemm_w8_workspace_bytes(m, n, k), 256), dtype=torch.uint8, device=DEV)
    X = dev_tensor(synth.outlier_activations(synth.stream(4, 91, 3), 1500, 2048, 0.005, 30.0), BF)
    w = dev_tensor(synth.bf16_round(synth.stream(4, 91, 4).uniform(0.2, 1.5, 2048)), BF)
    Yn = torch.empty_like(X)
    sn = torch.empty(2048, dtype=torch.float32, device=DEV)
    ws_n = torch.empty(max(R.rmm_rmsnorm_scored_workspace_bytes(1500, 2048), 256), dtype=torch.uint8, device=DEV)
    G = dev_tensor(synth.outlier_activations(synth.stream(4, 91, 5), 1500, 1000, 0.005, 30.0), BF)
    U = dev_tensor(synth.outlier_activations(synth.stream(4, 91, 6), 1500, 1000, 0.005, 30.0), BF)
    H = torch.empty_like(G)
    sh = torch.empty(1000, dtype=torch.float32, device=DEV)
    ws_h = torch.empty(max(R.rmm_swiglu_scored_workspace_bytes(1500, 1000), 256), dtype=torch.uint8, device=DEV)

    def chain():
        R.rmm_colnorm(A, out=s, ws=ws_c)
        R.rmm_topk(s, k, out=idx)
        R.rmm_gemm_w8(A, qd, scd, idx, k, out=Y, ws=ws_w)
        R.rmm_rmsnorm_scored(X, w, 1e-5, Y=Yn, scores=sn, ws=ws_n)
        R.rmm_swiglu_scored(G, U, H=H, scores=sh, ws=ws_h)

    _replay_matches(chain, [s, idx, Y, Yn, sn, H, sh])
