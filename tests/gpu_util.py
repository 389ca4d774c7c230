"""Shared helpers of the GPU tests: device inputs from the seeded generators."""
import sys

import numpy as np
import torch

import eec_inputs as I
from equivariant_edge_convolution_amd import binding as B

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_inputs(cfg):
    pos = torch.as_tensor(cfg.pos).to(DEV)
    species = torch.as_tensor(cfg.species).to(DEV)
    model = B.Model.from_arrays(cfg.model, DEV)
    return pos, species, model


def graph_for(cfg, pos, species):
    return B.build_neighbors(pos, cfg.box, cfg.model.cutoff, species, cfg.model.n_species)


def np_(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rms(x):
    return float(np.sqrt(np.mean(np.asarray(x, np.float64) ** 2)))
