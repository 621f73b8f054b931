"""Oracle prompt-lookup (n-gram) drafter.  TEST INFRASTRUCTURE ONLY.

Sangama, "Speculative decoding: correct, but slower (for now)": if the last 2-4
tokens of the text appeared earlier, guess the tokens that followed them then.
Readings where the page is silent: the longest suffix length is tried first;
among earlier occurrences the most recent one is used; up to k_max following
tokens are proposed, stopping at the end of the history.
"""


def propose(hist, min_n=2, max_n=4, k_max=8):
    """Return the list of proposed tokens (possibly empty)."""
    h = [int(t) for t in hist]
    N = len(h)
    for n in range(max_n, min_n - 1, -1):
        if N < n + 1:
            continue
        suffix = h[N - n:]
        for j in range(N - n - 1, -1, -1):          # most recent start first, j < N - n
            if h[j:j + n] == suffix:
                return h[j + n:min(j + n + k_max, N)]
    return []
