"""The five synthetic workloads: shapes, value distributions and seeds.

Shapes and distributions only; no approximate arithmetic. Each tensor has
its own seed, ``tensor_seed(config, id)``. The multiplier table of each
workload is named by (model, M, perturbation) and built elsewhere:
"exact" is the exact mantissa product, "mitchell" Mitchell's logarithmic
multiplier, and a perturbation is a +/-1 per-entry sign stream.
"""
from . import glorot_uniform, he_normal, normal, pm_one, tensor_seed, uniform, PERTURB_SEED


def lut_spec(config):
    """(model, M, perturbation or None) of a workload's multiplier table."""
    if config == 1:
        return "exact", 7, None
    if config == 4:
        return "exact", 8, pm_one(PERTURB_SEED, 1 << 16)
    return "mitchell", 7, None


def gemm_square(config, size):
    """A, B ~ N(0, 1), both size x size (workloads 1 and 4)."""
    A = normal(tensor_seed(config, 1), (size, size))
    B = normal(tensor_seed(config, 2), (size, size))
    return A, B


MLP_BATCH = 256
MLP_WIDTHS = (784, 1024, 1024, 10)


def mlp_tensors(batch=MLP_BATCH, widths=MLP_WIDTHS, config=2):
    """Per layer l: X_l ~ U(0,1) [batch x in], W_l Glorot-uniform [in x out],
    dY_l ~ N(0,1) [batch x out]."""
    layers = []
    for l in range(len(widths) - 1):
        fi, fo = widths[l], widths[l + 1]
        X = uniform(tensor_seed(config, 10 * l + 1), (batch, fi))
        W = glorot_uniform(tensor_seed(config, 10 * l + 2), fi, fo)
        dY = normal(tensor_seed(config, 10 * l + 3), (batch, fo))
        layers.append((X, W, dY))
    return layers


def mlp_gemms(batch=MLP_BATCH, widths=MLP_WIDTHS):
    """(name, transA, transB, m, n, k, A-name, B-name) of the 9 layer GEMMs:
    forward Y = X W, input gradient dX = dY W^T, weight gradient dW = X^T dY."""
    out = []
    for l in range(len(widths) - 1):
        fi, fo = widths[l], widths[l + 1]
        out.append((f"fwd{l}", 0, 0, batch, fo, fi, "X", "W"))
        out.append((f"dgrad{l}", 0, 1, batch, fi, fo, "dY", "W"))
        out.append((f"wgrad{l}", 1, 0, fi, fo, batch, "X", "dY"))
    return out


CONV_SHAPE = dict(N=128, H=32, W=32, C=64, K=64, R=3, S=3, stride=(1, 1), pad=(1, 1))


def conv_tensors(N=128, H=32, W=32, C=64, K=64, R=3, S=3, stride=(1, 1), pad=(1, 1), config=3):
    """X ~ N(0,1) NHWC, W He-normal RSCK (fan-in R*S*C), dY ~ N(0,1) NPQK."""
    P = (H + 2 * pad[0] - R) // stride[0] + 1
    Q = (W + 2 * pad[1] - S) // stride[1] + 1
    X = normal(tensor_seed(config, 1), (N, H, W, C))
    Wt = he_normal(tensor_seed(config, 2), (R, S, C, K), R * S * C)
    dY = normal(tensor_seed(config, 3), (N, P, Q, K))
    return X, Wt, dY


MHA_SHAPE = dict(batch=16, seq=512, d_model=768, heads=12)


def mha_tensors(batch=16, seq=512, d_model=768, config=5):
    """X ~ N(0,1) [batch*seq x d_model]; Wqkv [d_model x 3 d_model] and
    Wo [d_model x d_model] ~ N(0, 0.02**2)."""
    X = normal(tensor_seed(config, 1), (batch * seq, d_model))
    Wqkv = normal(tensor_seed(config, 2), (d_model, 3 * d_model), std=0.02)
    Wo = normal(tensor_seed(config, 3), (d_model, d_model), std=0.02)
    return X, Wqkv, Wo


def macs(config):
    """Approximate-MAC count of one pass of a workload."""
    if config == 1:
        return 64 ** 3
    if config == 4:
        return 8192 ** 3
    if config == 2:
        return sum(m * n * k for (_, _, _, m, n, k, _, _) in mlp_gemms())
    if config == 3:
        s = CONV_SHAPE
        return 3 * s["N"] * s["H"] * s["W"] * s["K"] * s["R"] * s["S"] * s["C"]
    if config == 5:
        b, t, d, h = MHA_SHAPE["batch"], MHA_SHAPE["seq"], MHA_SHAPE["d_model"], MHA_SHAPE["heads"]
        dh = d // h
        return b * t * 3 * d * d + 2 * b * h * t * t * dh + b * t * d * d
    raise ValueError(config)
