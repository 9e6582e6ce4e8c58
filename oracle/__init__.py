"""CPU oracle for the Talker MoE layer — test infrastructure, not part of the product.

Plain float64 numpy (``moe_ref``) and scalar pure-Python (``lab_scalar``)
statements of the layer, used only by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg.  The HIP library never imports or calls it.
"""
