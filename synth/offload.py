"""Placement of the two-layer offloaded decode workload: layer 0 entirely in
HBM, layer 1's queries and compressed keys in HBM and its K/V in pinned host
memory. Values come from the seeded generator; the compressed keys are built by
the ``compress`` callable the caller passes in (this module holds none of the
method's arithmetic)."""

from __future__ import annotations

from . import gpu as sg


def offload_layers(w, compress, device="cuda", chunk_B: int = 8):
    """(layer0, layer1) dicts of tensors for workload ``w`` (two layers).

    layer0: Q, F_self (same-layer Forecast), F_next (Forecast of layer 1's
    blocks), K, V, Kc.  layer1: Q, Kc, host_K, host_V.  Layer 1's compressed
    keys are built from its keys on the device, ``chunk_B`` sequences at a
    time, before the keys are placed in host memory.
    """
    import torch
    l0 = {name: sg.tensor(w.recipe(src, 0), w.shape(src), device)
          for name, src in (("Q", "Q"), ("F_self", "F_self"), ("F_next", "F"), ("K", "K"), ("V", "V"))}
    l0["Kc"] = compress(l0["K"])
    l1 = {"Q": sg.tensor(w.recipe("Q", 1), w.shape("Q"), device)}
    kshape = w.shape("K")
    kc1 = torch.empty(w.shape("Kc"), dtype=l0["Kc"].dtype, device=device)
    per_seq = kshape[1] * kshape[2] * kshape[3]
    buf = torch.empty((min(chunk_B, w.B),) + kshape[1:], dtype=l0["K"].dtype, device=device)
    for b0 in range(0, w.B, chunk_B):
        b1 = min(w.B, b0 + chunk_B)
        part = buf[: b1 - b0]
        sg.fill_(part, w.recipe("K", 1), kshape, start=b0 * per_seq)
        compress(part, out=kc1[b0:b1])
    del buf
    l1["Kc"] = kc1
    l1["host_K"] = sg.pinned_tensor(w.recipe("K", 1), kshape, device)
    l1["host_V"] = sg.pinned_tensor(w.recipe("V", 1), kshape, device)
    return l0, l1


def offload_stack(w, L: int, compress, device="cuda", chunk_B: int = 8, depth: int = 1):
    """Inputs of an L-layer offloaded decode step for workload ``w``: layer 0
    entirely in HBM (Q, F_self, F_next, K, V, Kc); layers 1 .. L-1 with Q and
    Kc in HBM, K/V in pinned host memory (host_K, host_V), and, except the
    last, F_next (the layer's Forecast of the next layer's blocks).

    With ``depth`` > 1 (Forecasts that look that many layers ahead) layer 0
    also gets F_ahead, the list of its Forecasts of layers 1 .. depth, and
    layer l >= 1 gets F_ahead, its Forecast of layer l + depth (if any)."""
    import torch
    layers = list(offload_layers(w, compress, device, chunk_B))
    kshape = w.shape("K")
    per_seq = kshape[1] * kshape[2] * kshape[3]
    for l in range(2, L):
        lay = {"Q": sg.tensor(w.recipe("Q", l), w.shape("Q"), device)}
        kc = torch.empty(w.shape("Kc"), dtype=layers[0]["Kc"].dtype, device=device)
        buf = torch.empty((min(chunk_B, w.B),) + kshape[1:], dtype=layers[0]["K"].dtype, device=device)
        for b0 in range(0, w.B, chunk_B):
            b1 = min(w.B, b0 + chunk_B)
            part = buf[: b1 - b0]
            sg.fill_(part, w.recipe("K", l), kshape, start=b0 * per_seq)
            compress(part, out=kc[b0:b1])
        del buf
        lay["Kc"] = kc
        lay["host_K"] = sg.pinned_tensor(w.recipe("K", l), kshape, device)
        lay["host_V"] = sg.pinned_tensor(w.recipe("V", l), kshape, device)
        layers.append(lay)
    for l in range(1, L - 1):
        layers[l]["F_next"] = sg.tensor(w.recipe("F", l), w.shape("F"), device)
    layers = layers[:L]
    if depth > 1:
        set_lookahead(w, layers, depth, device)
    return layers


def set_lookahead(w, layers: list, depth: int, device="cuda") -> None:
    """Give a stack the Forecast vectors of lookahead ``depth`` > 1 (replacing
    any earlier F_ahead): layer 0's F_ahead lists its Forecasts of layers
    1 .. depth (the first is F_next), layer l >= 1's is its Forecast of layer
    l + depth."""
    L = len(layers)
    for lay in layers:
        lay.pop("F_ahead", None)
    layers[0]["F_ahead"] = [layers[0]["F_next"]] + [sg.tensor(w.recipe("F", 0, j), w.shape("F"), device)
                                                    for j in range(2, min(depth, L - 1) + 1)]
    for l in range(1, L - depth):
        layers[l]["F_ahead"] = sg.tensor(w.recipe("F", l, depth), w.shape("F"), device)
