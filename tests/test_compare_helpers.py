"""Host checks of the comparison helpers the GPU parity tests rely on."""
import numpy as np

from gpu_util import scale_mismatches


def _b(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_scale_mismatches_normalisation_and_explanation():
    sr, cr = _b([1.0, 0.5, 2.0, 0.25]), _b([0.0078125, 0.015625, 0.03125])
    nodiff = np.zeros((4, 3), bool)
    allrows = np.ones(4, bool)
    assert scale_mismatches(sr, cr, sr, cr, nodiff, allrows) == (0, 0, 0)
    # another E: every sigma x2, every c /2, same steps sigma_i c_j
    assert scale_mismatches(_b([2.0, 1.0, 4.0, 0.5]), _b([0.00390625, 0.0078125, 0.015625]), sr, cr,
                            nodiff, allrows) == (0, 0, 0)
    # one column scale one bf16 step off, with a differing code in that column
    cg = _b([0.0078125, 0.015625 * (1 + 2 ** -7), 0.03125])
    d = nodiff.copy(); d[2, 1] = True
    assert scale_mismatches(sr, cg, sr, cr, d, allrows) == (1, 0, 1)
    # ... and without one: unexplained
    assert scale_mismatches(sr, cg, sr, cr, nodiff, allrows) == (1, 1, 1)
    # a row scale off, E shift on top, code difference in another row
    sg = _b([2.0, 1.0 * (1 + 2 ** -7), 4.0, 0.5])
    d = nodiff.copy(); d[0, 0] = True
    assert scale_mismatches(sg, _b([0.00390625, 0.0078125, 0.015625]), sr, cr, d, allrows) == (1, 1, 1)

    # two bf16 steps off
    cg2 = _b([0.0078125, 0.015625 * (1 + 2 ** -6), 0.03125])
    assert scale_mismatches(sr, cg2, sr, cr, nodiff, allrows)[2] == 2
