"""The threaded test helper gives the oracle's own results (rows are independent)."""
import numpy as np

import oracle
import par_oracle
import workloads


def test_threaded_forward_equals_oracle_forward():
    m, k, n = 3, 256, 301
    w = workloads.weights(9, n, k)
    x = workloads.activations(9, m, k)
    codes, packed, alpha = oracle.quantize_weights(w)
    xq, beta = oracle.quantize_act(x)
    acc_o, y_o = oracle.forward(xq, beta, packed, k, alpha)
    acc, y = par_oracle.forward(xq, beta, packed, k, alpha, threads=4)
    assert np.array_equal(acc, acc_o) and np.array_equal(y.view(np.uint32), y_o.view(np.uint32))
    ar = oracle.absmean_rows(w)
    bias = workloads.activations(9, 1, n)[0]
    acc_o, y_o = oracle.forward(xq, beta, oracle.pack(oracle.ternarize_rows(w, ar)), k, 0.0, bias=bias, alpha_rows=ar)
    acc, y = par_oracle.forward(xq, beta, oracle.pack(oracle.ternarize_rows(w, ar)), k, alpha_rows=ar, bias=bias,
                                threads=3)
    assert np.array_equal(acc, acc_o) and np.array_equal(y.view(np.uint32), y_o.view(np.uint32))
