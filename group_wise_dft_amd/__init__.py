"""Flash EQ-Linear for AMD MI355X (gfx950).

``group_wise_dft_amd.eqlinear``  torch binding of libeqlinear.so (C ABI in
                                 include/eqlinear.h)
``group_wise_dft_amd.workloads`` seeded synthetic workloads
``group_wise_dft_amd.build``     in-tree hipcc build of libeqlinear.so
"""
