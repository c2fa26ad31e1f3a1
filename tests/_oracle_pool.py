"""Oracle scores of a large packed prod database in chunks, spread over worker processes (CPU
only: this module imports numpy and the oracle, nothing that touches a GPU)."""

import numpy as np

import oracle


def _load(path):
    names = ("words", "qwords", "norms", "rnorms", "rmat", "smat", "q", "meta")
    return {k: np.load(f"{path}/{k}.npy", mmap_mode="r") for k in names}


def save_db(path, **arrays):
    """Writes the arrays prod_scores_all reads (one .npy each, so workers can memory-map them)."""
    import os
    os.makedirs(path, exist_ok=True)
    for k, v in arrays.items():
        np.save(f"{path}/{k}.npy", np.ascontiguousarray(v))


def _chunk_scores(args):
    path, lo, hi = args
    z = _load(path)
    d, bits = int(z["meta"][0]), int(z["meta"][1])
    rmat, smat, q = z["rmat"], z["smat"], z["q"]
    cb = oracle.codebook(d, bits)
    enc = oracle.EncodedProd(
        mse=oracle.EncodedMSE(idx=oracle.unpack_bits(np.asarray(z["words"][lo:hi]), d, bits), words=None,
                              norms=np.asarray(z["norms"][lo:hi], dtype=np.float64), y=None),
        z=oracle.unpack_bits(np.asarray(z["qwords"][lo:hi]), d, 1).astype(bool), qjl_words=None,
        gamma=np.asarray(z["rnorms"][lo:hi], dtype=np.float64), proj=None)
    return lo, oracle.scores_prod(q, enc, rmat, cb, smat)


def prod_scores_all(path, n, chunk=20000, workers=16):
    """Scores [nq, n] of the queries against every database row stored in the directory `path`
    by save_db (words, qwords, norms, rnorms, rmat, smat, q, meta = [d, bits])."""
    import multiprocessing as mp
    jobs = [(path, lo, min(n, lo + chunk)) for lo in range(0, n, chunk)]
    out = None
    with mp.get_context("spawn").Pool(workers) as pool:
        for lo, s in pool.imap_unordered(_chunk_scores, jobs):
            if out is None:
                out = np.empty((s.shape[0], n))
            out[:, lo:lo + s.shape[1]] = s
    return out
