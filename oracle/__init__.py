"""Oracle for the MFA decode step: plain, slow, fp64 CPU code.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
executes anything in this package. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It imports numpy (and the
Python standard library) and nothing from the GPU package.

What it computes, and from where
--------------------------------
The subject is Step-3's Multi-Matrix Factorization Attention (MFA), as
summarised on the page "Step-3 is Large yet Affordable: Model-system Co-design
for Cost-effective Decoding":

* §2 (Step-3 Model Card): each Transformer block has one attention; MFA puts a
  low-rank factorisation in the QK circuit to widen the number of attention
  heads while keeping the KV cache small.
* §5 (Model-System Co-design): arithmetic intensity 128 with an 8-bit KV cache,
  effective rank 16,384; KV quantisation raises arithmetic intensity.
* §6 (Non-Flagship Hardware Support): the attention stays memory-bandwidth bound.
* §7 (Implementation and Results): attention instances own the KV caches.

The pages give no equations. The readings taken here (each stated where it is
used) are: the query path is a down-projection, an RMSNorm with a gain vector,
and an up-projection split into H heads; all H heads attend to one shared K/V
head with softmax(q k^T / sqrt(d)) v over every cached token; the FP8 cache is
OCP e4m3 with one fp32 scale amax/448 per token per K and per V.

Modules
-------
``e4m3``   bit-level OCP e4m3 codec (decode by closed form, encode by nearest
           representable value with ties to even).
``mfa``    query projection, RMSNorm, paged gather, decode attention, split
           partials and their log-sum-exp combine, per-token FP8 quantisation.
``brute``  pure-Python loops for tiny cases (no numpy).
``layout`` the physical cache layout the library documents, written out
           independently, for bit-exact checks of the KV append.
``cost``   bytes and flop per cached token (the cost model of §4/§5).

Every function is pinned by ``tests/test_oracle.py`` to something other than
itself (closed forms, invariants, brute force, library routines on special
cases, figures printed on the pages).
"""
