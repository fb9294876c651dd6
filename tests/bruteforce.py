"""Literal pure-Python loops for tiny shapes (independent of the C oracle).

Written from the definition of a stride-1 causal 3-D convolution with zero
spatial padding (kh-1)/2, (kw-1)/2 and kt-1 causal front frames that are zero
or come from an explicit cache of previous frames.  Lists of Python ints, no
numpy arithmetic, so that nothing here shares a code path with the oracle.
"""


def conv_acc_bruteforce(xq, wq, cache=None):
    """xq: nested list [N][T][H][W][Cin] of ints; wq: [Cout][kt][kh][kw][Cin];
    cache: [N][kt-1][H][W][Cin] or None.  Returns [N][T][H][W][Cout] ints."""
    N = len(xq)
    T = len(xq[0])
    H = len(xq[0][0])
    W = len(xq[0][0][0])
    Cin = len(xq[0][0][0][0])
    Cout = len(wq)
    kt = len(wq[0])
    kh = len(wq[0][0])
    kw = len(wq[0][0][0])
    out = []
    for n in range(N):
        on = []
        for t in range(T):
            ot = []
            for h in range(H):
                oh = []
                for w in range(W):
                    ow = []
                    for co in range(Cout):
                        s = 0
                        for i in range(kt):
                            src_t = t + i - (kt - 1)
                            for j in range(kh):
                                src_h = h + j - (kh - 1) // 2
                                for l in range(kw):
                                    src_w = w + l - (kw - 1) // 2
                                    if not (0 <= src_h < H and 0 <= src_w < W):
                                        continue
                                    if src_t >= 0:
                                        pix = xq[n][src_t][src_h][src_w]
                                    elif cache is not None:
                                        pix = cache[n][src_t + kt - 1][src_h][src_w]
                                    else:
                                        continue
                                    wv = wq[co][i][j][l]
                                    for c in range(Cin):
                                        s += wv[c] * pix[c]
                        ow.append(s)
                    oh.append(ow)
                ot.append(oh)
            on.append(ot)
        out.append(on)
    return out
